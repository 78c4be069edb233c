// Grouped FP8 GEMMs over the expert-major pool, on gfx950 MFMA (v_mfma_f32_16x16x128_f8f6f4).
//
//   GEMM1 (gate_up): for pool block b of local expert le, G = A W1[le]^T over K = H, with A the pooled
//     FP8 rows.  Epilogue: h = silu(gate) * up, then per row and 128 columns s = max(amax, 1e-4)/448 and
//     q = e4m3fn(h * (1/s)), with 1/s the fp32 reciprocal, into the L2 pool ("Mega-MoE kernel code walkthrough: from Dispatch to WGMMA",
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
// GEMM2, the tile's pool metadata) arrive by LDS DMA (global_load_lds) into one of N = 3 LDS stages.
// The persistent work-group walks its (tile, K step) sequence as one stream.  Step s computes from
// registers that were read from LDS during step s-1; half-way through, it waits until stage s+1 has
// landed (vmcnt lets the N-2 youngest DMA groups stay in flight), barriers, refills its own stage with
// step s+N and reads stage s+1 into the second register set while its remaining MFMAs run.  The next
// tile's first steps load during the current tile's last ones.  Every step issues the same number of
// DMA instructions (past the end the last step is loaded again), so the wait count is a constant.  LDS rows are 128 bytes with the 16-byte chunks
// XOR-swizzled by row; the DMA lanes fetch the global chunk that belongs at their LDS position.
// Tiles map XCD-aware: consecutive work-groups of one XCD take neighbouring tiles of one expert (a few
// n tiles of all its pool blocks), which share A and B through that XCD's L2.  A stream-ordered launch
// looks up its work-group's tiles (block, n tile, expert) once, into an LDS table.
//
// The same pipeline also runs with MXFP4 weights (kFp4: e2m1 codes with UE8M0 exponents applied by the
// scaled MFMA) and BF16 tokens and weights (kBf16: two 16x16x32 bf16 MFMAs per fragment pair, no scales,
// no promotion, and a bf16 L2 pool).
#include <type_traits>

#include "mm_internal.h"
#include "route_impl.h"

namespace mm {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kWaves = 8;         // waves per work-group, 2 per SIMD
// LDS stages of the load pipeline (steps in flight = stages - 1); the pipeline code below holds for any
// count.  FP8 stages (48 or 40 KB) fit three times in the 160 KB of LDS.  MXFP4's smaller stages would
// allow four (BLOCK_M 128) or five (BLOCK_M 64), which measured no faster in same-box A/B runs.
constexpr int stages_of(int /*BM*/, bool /*fp4*/) { return 3; }

// MXFP4 weight fragment (16 rows x 128 K as e2m1, 16 bytes per lane) times an FP8 token fragment; the
// weight rows' UE8M0 exponents come in through the MFMA's A-scale operand (byte 0 of `sa`, one per lane:
// its row and its 32-value K block), the token side is unscaled (127 = 2^0).
__device__ __forceinline__ v4f mfma_fp4w(const v4i& a, const v8i& b, uint32_t sa, const v4f& c) {
    const v8i aw = __builtin_shufflevector(a, v4i{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw, b, c, 4, 0, 0, (int)sa, 0, 127);
}

// BF16 x BF16: a 32-byte fragment (16 bf16 values of lane group g's K range) feeds two 16x16x32 MFMAs,
// its first and second 16 bytes; both operands split alike, so their K indices pair up.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v4f mfma_bf16_pair(const v8i& a, const v8i& b, v4f c) {
    const v4i a0 = __builtin_shufflevector(a, a, 0, 1, 2, 3), a1 = __builtin_shufflevector(a, a, 4, 5, 6, 7);
    const v4i b0 = __builtin_shufflevector(b, b, 0, 1, 2, 3), b1 = __builtin_shufflevector(b, b, 4, 5, 6, 7);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a0), __builtin_bit_cast(v8bf, b0), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a1), __builtin_bit_cast(v8bf, b1), c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
    // scale operands 0 select the unscaled v_mfma_f32_16x16x128_f8f6f4; format 0 = FP8 e4m3
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16-byte chunk c of a 128-byte LDS row r sits at position c ^ (r & 7) ^ ((r >> 3) & 1): the 16 rows
// of one fragment read land in 16 different 16-byte bank slots whether the LDS serves 8 or 16 lanes of a
// 128-bit read per cycle.
__device__ __forceinline__ int swz_chunk(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }
// 64-byte rows (MXFP4 weights, four 16-byte chunks): chunk c of row r at c ^ ((r >> 1) & 3).  Measured
// with the LDS bank-conflict counter: this leaves the fragment reads conflict-free, while also flipping
// with row bit 3 (as the 128-byte rows do) stalled 20% of the LDS-active cycles, as did the plain layout.
__device__ __forceinline__ int swz4_chunk(int r, int c) { return c ^ ((r >> 1) & 3); }
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + (swz_chunk(r, c) << 4); }

// Fragment of 16 rows x 128 K bytes for one MFMA operand: lane l takes row (l & 15) and the 32 bytes
// [32*(l>>4), +32).  A and B use the same lane -> K mapping, so the product sums every K exactly once.
// lo / hi point at the lane's two 16-byte chunks in the first fragment row block; fragments whose first
// row differs by a multiple of 16 (and other stages) sit at a constant byte offset from them, since the
// swizzle depends on the row's low four bits only.
__device__ __forceinline__ v8i load_frag(const uint8_t* lo, const uint8_t* hi, int off) {
    const v4i a = *reinterpret_cast<const v4i*>(lo + off);
    const v4i b = *reinterpret_cast<const v4i*>(hi + off);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
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

// Two fp32 -> two bf16 (round to nearest even) in one word, the first value in the low half.
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
}

// 4x4 transpose of (register i, lane row r = lane / 16): afterwards register i of row r holds what
// register r of row i held.  permlane32_swap exchanges the upper two rows of its first operand with
// the lower two of its second; permlane16_swap the odd rows of the first with the even rows of the
// second.
__device__ __forceinline__ void transpose4_rows(uint32_t (&R)[4]) {
    const auto s02 = __builtin_amdgcn_permlane32_swap(R[0], R[2], false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(R[1], R[3], false, false);
    const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
    const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
    R[0] = s01[0];
    R[1] = s01[1];
    R[2] = s23[0];
    R[3] = s23[1];
}
// The value of lane l ^ 1 (DPP quad permutation 1, 0, 3, 2).
__device__ __forceinline__ uint32_t swap_adjacent(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ v4u swap_adjacent(v4u v) {
    return v4u{swap_adjacent(v[0]), swap_adjacent(v[1]), swap_adjacent(v[2]), swap_adjacent(v[3])};
}

// LDS DMA: every lane copies 16 bytes from base + off (or 4 bytes from its own address) to LDS at
// dst + lane * size (dst and base wave-uniform, off per lane).  Inline asm: the waits for these writes are placed by hand
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
// The same with the non-temporal hint, for data read once (the caches keep it at low priority)
__device__ __forceinline__ void dma16_nt(const void* base, uint32_t off, const void* dst) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(off), "s"(base), "s"(lds_addr(dst)) : "memory", "m0");
}
// 4 bytes per lane from a per-lane address (every lane active)
__device__ __forceinline__ void dma4_lane(const void* src, const void* dst) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :: "v"(src), "s"(lds_addr(dst)) : "memory", "m0");
}
// 4 bytes per active lane from base + off (base wave-uniform, off per lane) to LDS at dst + lane * 4
__device__ __forceinline__ void dma4(const void* base, uint32_t off, const void* dst) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(off), "s"(base), "s"(lds_addr(dst)) : "memory", "m0");
}
// 4 bytes per active lane with the cache policy of a device-scope atomic load (sc1), for schedule words
// that other work-groups of the launch update
__device__ __forceinline__ void dma4_coherent(const void* src, const void* dst) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off sc1"
                 :: "v"(src), "s"(lds_addr(dst)) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are outstanding and its LDS reads have
// returned, then barrier.  The compiler's __syncthreads would drain every LDS DMA in flight; this keeps
// the younger stage loading.
template <int N>
__device__ __forceinline__ void wait_stage_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Wait until every vector-memory access of this wave, stores included, has completed.
__device__ __forceinline__ void wait_all_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }


// ---------------------------------------------------------------- launches that hand data over inside
// Two schedules let a kernel consume rows that other work-groups of the same launch produce:
//   FILL_IN_GEMM1: GEMM1's work-groups first pull the pool rows themselves, with the per-block arrival
//     count of "Mega-MoE notes, part 2: index table and pull" (2.6), and a GEMM1 tile waits for its own
//     block's count before its first load;
//   ONE_GEMM_LAUNCH: GEMM1 and GEMM2 run in one persistent launch, and a GEMM2 tile waits for the count
//     of finished GEMM1 n tiles of its pool block ("MoE fused operators", DeepGEMM part, 2: the L2 GEMM
//     waits per m block for its L1 n tiles).
// Every hand-over stays inside one XCD.  The work-groups of XCD x (read from the hardware register
// XCC_ID) own a contiguous range of pool blocks: they pull those blocks' rows, run their GEMM1 tiles and
// then their GEMM2 tiles.  The producer's stores reach that XCD's L2 (s_waitcnt vmcnt(0)) before a
// relaxed device-scope atomic counts them, and the consumer's loads are served by the same L2, which is
// the coherence point of all CUs of an XCD; no L2 writeback or invalidation is needed.  A work-group
// takes its slot (XCD, blockIdx / 8) with an atomic bit: if the hardware ever placed two work-groups in
// one slot (dispatch not round-robin over the eight XCDs), MEGA_MOE_STATUS_PLACEMENT is latched.
// Consumers read the count through a one-lane probe DMA issued with every K step (so the check costs
// no pipeline drain) and fall back to bounded polls; nothing waits on work that no running wave holds.
constexpr int kXcds = 8;
constexpr int kFillRows = 8;                   // rows per code unit
constexpr long long kSpinTicks = 200000000;    // ~2 s of the 100 MHz constant clock

template <int BM>
struct FillUnits {
    static constexpr int rows = BM / kFillRows, scales = BM / 64, per_block = rows + scales;
};

// The XCD this wave runs on (HW_REG_XCC_ID, bits 3:0).
__device__ __forceinline__ int xcc_id() { return (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u); }

__device__ __forceinline__ uint32_t claim_unit(uint32_t* ctr, int lane) {
    uint32_t u = 0;
    if (lane == 0) u = atomicAdd(ctr, 1u);
    return __builtin_amdgcn_readfirstlane(u);
}

// device-scope relaxed load of a schedule word, one per wave
__device__ __forceinline__ uint32_t sched_peek(const uint32_t* ptr) {
    return __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(const_cast<uint32_t*>(ptr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Codes of pool rows row0 .. row0+7 (one block).  Lane l copies chunk columns l, l+64, ... of every
// row, two columns of all 8 rows per batch, all loads of a batch before its stores and no branch
// between them; chunk indices past a row's end are clamped to its last chunk (the same bytes are
// copied twice).  Padding rows and rows naming no valid token read token 0 and store zeros.
template <int BM>
__device__ __forceinline__ void fill_code_unit(const Params& p, int row0, int lane) {
    const int H16 = p.H >> 4, J = (H16 + 63) >> 6, SF = p.H >> 7;
    const int b = row0 / BM, i0 = row0 - b * BM;
    const char* src[kFillRows];
    char* dst[kFillRows];
    bool ok[kFillRows];
    bool bad = false;
#pragma unroll
    for (int r = 0; r < kFillRows; ++r) {
        const uint32_t ms = p.pool_meta[(size_t)(row0 + r) * 3], mt = p.pool_meta[(size_t)(row0 + r) * 3 + 1];
        ok[r] = ms < (uint32_t)p.S && mt < (uint32_t)p.T_max;
        bad |= !ok[r] && ms != kMetaPad;
        src[r] = reinterpret_cast<const char*>(p.x + (ok[r] ? ((size_t)ms * p.T_max + mt) * p.H : 0));
        dst[r] = reinterpret_cast<char*>(p.pool_x + (size_t)b * SF * BM * 128 + (size_t)(i0 + r) * 128);
    }
    if (bad && lane == 0) atomicOr(p.status, MEGA_MOE_STATUS_BAD_LAYOUT);
    // two chunk columns of all 8 rows per batch: 16 loads in flight per lane
    for (int j0 = 0; j0 < J; j0 += 2) {
        v4i v[2][kFillRows];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int c = min(min(j0 + jj, J - 1) * 64 + lane, H16 - 1);
#pragma unroll
            for (int r = 0; r < kFillRows; ++r) v[jj][r] = *reinterpret_cast<const v4i*>(src[r] + (size_t)c * 16);
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int c = min(min(j0 + jj, J - 1) * 64 + lane, H16 - 1);
            const size_t off = (size_t)(c >> 3) * (BM * 128) + (c & 7) * 16;
            const v4i z = {0, 0, 0, 0};
#pragma unroll
            for (int r = 0; r < kFillRows; ++r) *reinterpret_cast<v4i*>(dst[r] + off) = ok[r] ? v[jj][r] : z;
        }
    }
}

// Scales of the 64 pool rows row0 .. row0+63 (lane = row), block-major: K block k of row i of block b
// at pool_sf[(b*SF + k)*BM + i], so each K block's 64 values are one 256-byte store.
template <int BM>
__device__ __forceinline__ void fill_scale_unit(const Params& p, int row0, int lane) {
    const int SF = p.H >> 7;
    const int row = row0 + lane;
    const uint32_t ms = p.pool_meta[(size_t)row * 3], mt = p.pool_meta[(size_t)row * 3 + 1];
    const bool ok = ms < (uint32_t)p.S && mt < (uint32_t)p.T_max;
    const float2* ssf = reinterpret_cast<const float2*>(p.x_sf + (ok ? ((size_t)ms * p.T_max + mt) * SF : 0));
    const int b = row / BM, i_in = row - b * BM;
    float* dsf = p.pool_sf + (size_t)b * SF * BM + i_in;
    for (int k0 = 0; k0 < SF; k0 += 32) {     // SF is even (H is a multiple of 256)
        float2 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = ssf[min(k0 / 2 + u, SF / 2 - 1)];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int k = min(k0 + 2 * u, SF - 2);
            dsf[(size_t)k * BM] = ok ? v[u].x : 0.f;
            dsf[(size_t)(k + 1) * BM] = ok ? v[u].y : 0.f;
        }
    }
}

// Pull the rows of pool blocks [blo, bhi) in units, in pool order: per block, BM/8 units of 8 rows
// (codes), then BM/64 units of 64 rows (scales, written block-major as whole 256-byte lines).  A wave
// claims a unit with one atomic on its XCD's counter (the next claim is issued before the copy, so its
// latency hides under it), copies it, waits until its stores have completed and only then counts it in
// its block's arrival word.
template <int BM>
__device__ __forceinline__ void fill_blocks(const Params& p, int blo, int bhi, uint32_t* claim, int lane) {
    using U = FillUnits<BM>;
    const uint32_t total = (uint32_t)(bhi - blo) * U::per_block;
    uint32_t u = claim_unit(claim, lane);
    while (u < total) {
        const uint32_t next = claim_unit(claim, lane);
        const int b = blo + (int)(u / U::per_block), v = (int)(u % U::per_block);
        if (v < U::rows) fill_code_unit<BM>(p, b * BM + v * kFillRows, lane);
        else fill_scale_unit<BM>(p, b * BM + (v - U::rows) * 64, lane);
        wait_all_vm();
        if (lane == 0) atomicAdd(p.sched + kSchedArrival + b, 1u);
        u = next;
    }
}

// Bounded spin (per wave) until *word reaches `target`; polls are spaced by a sleep.  A wait longer than
// kSpinTicks latches TIMEOUT and gives up: never expected, it keeps a broken schedule from hanging the
// GPU.  MEGA_MOE_FLAG_DEBUG_FORCE_TIMEOUT makes every wait give up as soon as the clock moves, so tests
// reach that path from the host.
// Returns whether the target was reached.  kForceable: MEGA_MOE_FLAG_DEBUG_FORCE_TIMEOUT applies.
template <bool kForceable = true>
__device__ __forceinline__ bool spin_until(const Params& p, const uint32_t* word, uint32_t target, int lane) {
    const bool force = kForceable && (p.flags & MEGA_MOE_FLAG_DEBUG_FORCE_TIMEOUT);
    if (!force && sched_peek(word) >= target) return true;
    const long long limit = force ? 0 : kSpinTicks;
    const long long t0 = wall_clock64();
    while (force || sched_peek(word) < target) {
        if (wall_clock64() - t0 > limit) {
            if (lane == 0) atomicOr(p.status, MEGA_MOE_STATUS_TIMEOUT);
            return false;
        }
        __builtin_amdgcn_s_sleep(32);
    }
    return true;
}

// Every work-group takes an exit ticket after its last access to the schedule words (its atomics have
// completed); the last one returns them to zero, so every forward starts from a clean schedule.
__device__ __forceinline__ void sched_exit(const Params& p, int nblocks, int tid) {
    __shared__ int sLast;
    wait_all_vm();
    __syncthreads();
    if (tid == 0) sLast = atomicAdd(p.sched + kSchedExit, 1u) == gridDim.x - 1;
    __syncthreads();
    if (sLast) {
        auto zero = [](uint32_t* w) { __hip_atomic_store(w, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
        for (int i = tid; i < nblocks; i += blockDim.x) {
            zero(p.sched + kSchedArrival + i);
            zero(p.sched + kSchedArrival + p.max_blocks + i);
        }
        if (tid < kSchedArrival) zero(p.sched + tid);
    }
}

template <int V>
using ic = std::integral_constant<int, V>;

#ifndef MM_ROT_J
#define MM_ROT_J 2
#endif
#ifndef MM_ROT_N
#define MM_ROT_N 2
#endif

// LDS of a work-group.  Each array is a function-local __shared__ variable of a template that does not
// depend on which GEMM runs, so the two phases of a launch that runs both GEMMs share it, and each
// array keeps its own symbol (the allocator places them as separately declared arrays).
template <int BM, int NW, bool kFp4>
struct GemmLds {
    static constexpr int kStages = stages_of(BM, kFp4);
    static constexpr int WRB = kFp4 ? 64 : 128;     // weight bytes per row and K step
    __device__ __forceinline__ static auto& sA() {
        __shared__ __attribute__((aligned(1024))) uint8_t v[kStages][BM * 128];
        return v;
    }
    __device__ __forceinline__ static auto& sB() {
        __shared__ __attribute__((aligned(1024))) uint8_t v[kStages][256 * WRB];
        return v;
    }
    // MXFP4: per stage and wave, the UE8M0 exponents of the wave's 64 weight rows (4 bytes = 4 K blocks)
    __device__ __forceinline__ static auto& sWs() {
        __shared__ __attribute__((aligned(16))) uint32_t v[kStages][kFp4 ? NW * 64 : 1];
        return v;
    }
    // per stage and wave, 64 dwords written by one DMA: [0, BM/NW) token scales of rows
    // wave*BM/NW + l, then the wave's two weight-block scales, then (GEMM2) the rows' scatter targets
    __device__ __forceinline__ static auto& sSmall() {
        __shared__ __attribute__((aligned(16))) uint32_t v[kStages][NW * 64];
        return v;
    }
    // per stage and wave, the schedule word of the next tile's block (probe DMA)
    __device__ __forceinline__ static auto& sProbe() {
        __shared__ __attribute__((aligned(16))) uint32_t v[kStages][NW];
        return v;
    }
    __device__ __forceinline__ static auto& sRed() {
        __shared__ float v[BM][NW / 2];
        return v;
    }
    __device__ __forceinline__ static auto& sOff() {
        __shared__ int v[MEGA_MOE_MAX_LOCAL_EXPERTS + 2];
        return v;
    }
    // the first kTileTab tiles of the work-group's run: {pool block, n tile, local expert, first K block}
    static constexpr int kTileTab = 128;
    __device__ __forceinline__ static auto& sTile() {
        __shared__ __attribute__((aligned(16))) uint4 v[kTileTab];
        return v;
    }
};

// Which pool blocks a work-group's tiles come from, and which of their tiles it takes: tiles first,
// first + stride, ... of the blocks [blo, bhi), numbered as described at tile_of.
struct TilePlan {
    int blo, bhi, first, stride;
};

// The wait of a phase's tiles before their first load: none, the fill units of the tile's block, or
// the GEMM1 n tiles of the tile's block.
enum { kWaitNone = 0, kWaitFill = 1, kWaitGemm1 = 2 };

// One GEMM over the plan's tiles.  Work-group: NW waves in a 2 x NW/2 grid over the BM x 256 tile.
// kStreamW: the weight DMA carries the non-temporal hint, for launches where each weight chunk is read
// by one tile only (about one pool block per expert, as at decode); where several blocks of an expert
// share a weight chunk through L2 (prefill) the hint costs 11% and is not used.  kFp4: MXFP4 weights
// (two e2m1 codes per byte, 64-byte rows per K step, UE8M0 exponents per 32 K applied by the MFMA's
// scale operand).  kWait: what a tile waits for before its first load.  kPublish (GEMM1): after a
// tile's stores have completed, count the tile in its block's GEMM1 word.
template <int BM, int NW, bool kGemm1, bool kStreamW, bool kFp4, int kWait, bool kPublish, bool kXcd,
          bool kBf16 = false>
__device__ __forceinline__ void gemm_phase(const Params& p, const TilePlan& plan, int nblocks) {
    using Lds = GemmLds<BM, NW, kFp4>;
    auto& sA = Lds::sA();
    auto& sB = Lds::sB();
    auto& sWs = Lds::sWs();
    auto& sSmall = Lds::sSmall();
    auto& sProbe = Lds::sProbe();
    auto& sRed = Lds::sRed();
    auto& sOff = Lds::sOff();
    constexpr int NWN = NW / 2;                 // compute waves along the weight (N) side
    constexpr int TM = BM / 32;                 // 16-token subtiles per wave (wave covers BM/2 tokens)
    constexpr int WROWS = 256 / NWN;            // weight rows per wave
    constexpr int WN = WROWS / 16;              // 16-row weight subtiles per wave
    constexpr int HC = WROWS / 2;               // GEMM1: output columns per wave (gate + up halves)
    constexpr int NMF = TM * WN;                // MFMAs per wave and K step
    constexpr int A_INS = BM / (8 * NW);        // 1 KB A DMA instructions per wave and step
    constexpr int WRB = GemmLds<BM, NW, kFp4>::WRB;
    constexpr int B_INS = (256 * WRB / 1024) / NW;   // 1 KB B DMA instructions per wave and step
    constexpr int SA_LANES = BM / NW;           // token rows whose scale (and GEMM2 target) a wave loads
    // The small DMA: a phase whose tiles do not wait loads its token scales, weight-block scales and
    // (GEMM2) scatter targets with one instruction from per-lane addresses (kLaneSmall); a phase whose
    // tiles wait needs those registers for its per-tile check and uses one exec-masked instruction per
    // kind of word from wave-uniform bases instead (one more DMA per step, two more with GEMM2).
    constexpr bool kLaneSmall = kWait == kWaitNone;
    // per step: A and B chunks, the small DMA, (MXFP4) the wave's weight-row exponents and (kWait) the
    // probe of the next tile's word.  BF16 has no scales: with kWait only the targets and the probe.
    constexpr int DMA_PER_STEP = A_INS + B_INS + (kBf16 && !kLaneSmall ? 0 : 1) + (kFp4 ? 1 : 0) +
                                 (kLaneSmall ? 0 : (kFp4 || kBf16 ? 0 : 1) + (kGemm1 ? 0 : 1) + 1);
    // global stores every wave issues in a GEMM2 tile's epilogue: two per 16-token group
    constexpr int kEpiStores = 2 * TM;
    // K-start rotation per block within the expert and per n tile (see the issue side below); it
    // shortens the down GEMM and not the gate_up GEMM, whose tiles are 3.5 times longer
    constexpr bool kRotate = !kGemm1;
    constexpr int kRotJ = MM_ROT_J, kRotN = MM_ROT_N;
    static_assert(A_INS >= 1 && B_INS >= 1 && 2 * SA_LANES + 2 <= 64, "tile shape");
    static_assert(TM * 32 == BM && WN * 16 == WROWS, "tile shape");
    static_assert(kGemm1 || kWait != kWaitFill, "the fill feeds GEMM1 only");
    static_assert(kGemm1 || !kPublish, "GEMM1 publishes its tiles");
    // BF16 x BF16: no scales, K steps of 64 values (128 bytes like FP8); stream-ordered tiles, or both
    // GEMMs in one launch (no pull inside it)
    static_assert(!kBf16 || (!kFp4 && kWait != kWaitFill), "BF16 schedule");
    constexpr int kStages = GemmLds<BM, NW, kFp4>::kStages;
    constexpr int kInFlight = (kStages - 2) * DMA_PER_STEP;   // at mid-step: the steps after the next one
    static_assert((kStages - 1) * DMA_PER_STEP + kEpiStores < 64, "vmcnt immediate");

    // The thread index is laundered, so the per-lane values of the phase are formed here: a launch that
    // runs phases in a loop (expert waves) would otherwise keep them live across every phase.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = (wave / NWN) & 1, wn = wave % NWN;
    const int rr = lane & 15, g = lane >> 4;
    const int Kdim = kGemm1 ? p.H : p.I;
    const int KB = kBf16 ? Kdim >> 6 : Kdim >> 7;
    const int NT = kGemm1 ? (p.I >> 7) : (p.H >> 8);
    const int ntiles = (plan.bhi - plan.blo) * NT;
    if (plan.first >= ntiles) return;
    const int my_tiles = (ntiles - 1 - plan.first) / plan.stride + 1;
    const int nsteps = my_tiles * KB;
    const int nseg = p.El + p.nsh;              // pool segments: routed experts, then the shared one

    // Tile t of the plan -> pool block, n tile and local expert.  With c[le] = the offset of expert le
    // clipped to the plan's blocks (relative to blo), tiles are numbered expert by expert (expert le
    // owns tiles [c[le]*NT, c[le+1]*NT)), inside an expert n tile by n tile, then block by block.  A
    // run of 32 consecutive tiles (one XCD's share of a round) then covers about four n tiles of every
    // block of one expert: the blocks' A chunks and the n tiles' W chunks are shared through that
    // XCD's L2, each W tile is fetched by one or two XCDs and each A block about NT/4 times.
    auto clip = [&](int i) { return kXcd ? min(max(sOff[i], plan.blo), plan.bhi) - plan.blo : sOff[i]; };
    auto tile_search = [&](int j, int& b, int& nt, int& le) __attribute__((always_inline)) {
        const int t = plan.first + j * plan.stride;
        const int vb = t / NT;
        int lo = 0, hi = nseg;              // the expert with c[le] <= vb < c[le+1]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (clip(mid) <= vb) lo = mid; else hi = mid;
        }
        le = lo;
        const int b0 = clip(lo), nb = max(clip(lo + 1) - b0, 1);
        const int u = t - b0 * NT;
        nt = u / nb;
        b = plan.blo + b0 + (u - nt * nb);
    };
    // The search costs a chain of dependent LDS reads and an integer division, and every wave of the
    // work-group runs it at the same step of a tile change, so the matrix cores would idle meanwhile.
    // The work-group's first kTileTab tiles are therefore looked up once here, one tile per thread
    // (stream-ordered launches; the in-launch schedules have no registers to spare for it).
    auto& sTile = Lds::sTile();
    constexpr int kTileTab = kXcd ? 0 : Lds::kTileTab;
    // The K-start rotation of a tile (kRotate, see the issue side below): its block within the expert
    // and its n tile give the first K block, jb*kRotJ + nt*kRotN mod KB.
    auto rot_start = [&](int b, int nt, int le) {
        int kc = kRotJ * (b - sOff[le]) + kRotN * nt;
        while (kc >= KB) kc -= KB;
        return kc;
    };
    if constexpr (kTileTab > 0) {
        for (int j = tid; j < min(my_tiles, kTileTab); j += NW * 64) {
            int b, nt, le;
            tile_search(j, b, nt, le);
            b = min(max(b, 0), nblocks - 1);
            nt = min(max(nt, 0), NT - 1);
            sTile[j] = uint4{(uint32_t)b, (uint32_t)nt, (uint32_t)le, (uint32_t)(kRotate ? rot_start(b, nt, le) : 0)};
        }
        __syncthreads();
    }
    // kc: the tile's first K block when the table holds it, else -1
    auto tile_of = [&](int j, int& b, int& nt, int& le, int& kc) __attribute__((always_inline)) {
        if (kTileTab > 0 && (unsigned)j < (unsigned)kTileTab) {
            const uint4 v = sTile[j];
            b = (int)v.x;
            nt = (int)v.y;
            le = (int)v.z;
            kc = (int)v.w;
        } else {
            tile_search(j, b, nt, le);
            kc = -1;
        }
        // wave-uniform by construction; the offsets come from LDS, so say so for the scalar DMA bases
        b = __builtin_amdgcn_readfirstlane(min(max(b, 0), nblocks - 1));   // inconsistent offsets only
        nt = __builtin_amdgcn_readfirstlane(min(max(nt, 0), NT - 1));
        le = __builtin_amdgcn_readfirstlane(le);
        kc = __builtin_amdgcn_readfirstlane(kc);
    };
    // A (pool or L2 pool) and W (packed weights) are tiled: the K step kb of block b is the contiguous
    // BM x 128 chunk at a_base(b) + kb*BM*128, that of n tile nt of expert le the 256 x 128 chunk at
    // w_base(le, nt) + kb*256*128 (for GEMM1 its rows are the 128 gate rows, then the 128 up rows)
    auto a_base = [&](int b) { return (kGemm1 ? p.pool_x : p.l2_x) + (size_t)b * KB * BM * 128; };
    auto w_base = [&](int le, int nt) {
        return (kGemm1 ? p.w1 : p.w2) + ((size_t)le * NT + nt) * KB * (256 * WRB);
    };

    // per-lane DMA offsets (fixed for the whole phase)
    uint32_t a_off[A_INS], b_off[B_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        const int r = (i * NW + wave) * 8 + (lane >> 3), p = swz_chunk(r, lane & 7);
        // LDS position p of row r holds token chunk c.  Against MXFP4 weights a lane reads its token
        // row's chunks g and g + 4 (the hardware's K order for that MFMA); those are stored at the
        // positions the FP8 path reads as chunks 2g and 2g + 1, whose reads are free of bank conflicts
        // (reading chunks g and g + 4 of the plain layout stalled 20% of the LDS-active cycles).
        const int c = kFp4 ? ((p & 1) ? (p >> 1) + 4 : (p >> 1)) : p;
        // the L2 pool stores a K block as four 32-byte column quarters of BM rows each
        a_off[i] = kGemm1 ? r * 128 + c * 16 : (c >> 1) * (BM * 32) + r * 32 + (c & 1) * 16;
    }
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
        const int r = (i * NW + wave) * 8 + (lane >> 3), c = swz_chunk(r, lane & 7);
        if constexpr (kFp4) {
            const int r4 = (i * NW + wave) * 16 + (lane >> 2), c4 = swz4_chunk(r4, lane & 3);
            b_off[i] = r4 * 64 + c4 * 16;
        } else {
            b_off[i] = r * 128 + c * 16;
        }
    }
    // The small DMA fills the wave's 64 dwords of sSmall with one exec-masked instruction per kind of
    // word, each from a wave-uniform base: the token scales (lanes [0, SA_LANES): rows
    // wave*SA_LANES + l), the two weight-block scales (lanes SA_LANES and SA_LANES + 1; FP8 weights) and,
    // for GEMM2, the scatter targets of the same rows (lanes SA_LANES + 2 ..).  A lane's byte offset
    // from its kind's base is fixed for the phase.
    // kLaneSmall: lane role in the one small DMA (token scale of row wave*SA_LANES + l, weight-block
    // scale j, or (GEMM2) scatter target of row wave*SA_LANES + l; spare lanes, and with MXFP4 weights
    // the two weight-scale lanes, repeat lane 0's load) and the bytes its address advances per K step
    // (token scales are block-major, BM per K block; weight scales K-contiguous)
    // (BF16: no scales; every lane loads a scatter target, its own row's in the GEMM2 target lanes and
    // the wave's first row's otherwise)
    const int sm_role = kBf16 ? 2 : lane < SA_LANES ? 0 : lane < SA_LANES + 2 ? (kFp4 ? 3 : 1)
                      : (!kGemm1 && lane < 2 * SA_LANES + 2) ? 2 : 3;
    const bool tg_row = (unsigned)(lane - SA_LANES - 2) < (unsigned)SA_LANES;
    const int sm_row = wave * SA_LANES + (kBf16 ? (tg_row ? lane - SA_LANES - 2 : 0)
                                                : sm_role == 0 ? lane : sm_role == 2 ? lane - SA_LANES - 2 : 0);
    const uint32_t sm_inc = sm_role == 2 ? 0u : sm_role == 1 ? 4u : (uint32_t)(BM * 4);
    const bool sc_lane = lane < SA_LANES;
    const bool ws_lane = !kFp4 && (unsigned)(lane - SA_LANES) < 2u;
    const bool tg_lane = !kGemm1 && (unsigned)(lane - SA_LANES - 2) < (unsigned)SA_LANES;
    const uint32_t sm_off = ws_lane ? (kGemm1 && lane == SA_LANES + 1 ? (uint32_t)((p.I >> 7) * KB * 4) : 0u)
                                    : (uint32_t)(wave * SA_LANES + (sc_lane ? lane : max(lane - SA_LANES - 2, 0))) * 4u;

    // kWait: the words the tiles wait on (per pool block) and the count that completes a block
    const uint32_t* wait_words = p.sched + kSchedArrival + (kWait == kWaitGemm1 ? p.max_blocks : 0);
    const uint32_t wait_target = kWait == kWaitFill ? (uint32_t)FillUnits<BM>::per_block : (uint32_t)(p.I >> 7);

    // Issue side: the next step to load, tile ij, its ikb-th K step, K block ikc.  With kRotate a tile
    // walks its K blocks from a start that depends on its block and n tile, wrapping around: the
    // work-groups that share a W chunk (same n tile, different blocks) or an A chunk (same block,
    // different n tiles) then ask L2 for it a few steps apart instead of all at once, so one of them
    // takes the miss and the others hit.  The base pointers advance by one K block per issue.
    int ij = 0, ikb = 0, ikc = 0;
    const uint8_t* iA;
    const uint8_t* iW;
    const uint8_t* iSm;     // kLaneSmall: per lane
    const uint8_t* iWsl;    // kLaneSmall, MXFP4: per lane, the exponent word of this lane's weight row
    const uint8_t* iSc;     // the step's token scales (block-major: BM per K block)
    const uint8_t* iWsc;    // (FP8) the tile's first weight-block scale of the step (K-contiguous)
    const uint8_t* iDst;    // (GEMM2) the scatter targets of the tile's rows
    const uint8_t* iWs;     // (MXFP4) the exponent words of the step's 256 weight rows
    const uint32_t* iProbe = wait_words;    // kWait: the schedule word of the next tile's block
    // MXFP4: the tile row whose exponents this lane loads, fragment lane >> 4, row lane & 15 (the rows
    // the wave's weight fragments cover, in the order they are read back; 32 consecutive rows per half
    // wave, so one step's exponent load is two 128-byte runs)
    const int ws_tr = kGemm1 ? wn * 32 + ((lane >> 4) < 2 ? 0 : 128) + ((lane >> 4) & 1) * 16 + (lane & 15)
                             : wn * WROWS + (lane >> 4) * 16 + (lane & 15);
    const uint32_t ws_off = (uint32_t)ws_tr * 4u;
    // landed: the stage whose DMA landed last (-1 in the prologue)
    auto set_issue_tile = [&](int landed) __attribute__((always_inline)) {
        int b, nt, le, kc;
        tile_of(ij, b, nt, le, kc);
        if constexpr (kWait != kWaitNone) {
            // The tile's block is complete before its first load.  The probe DMA of the steps issued
            // for the previous tile read this block's word: the stage that landed last holds its value
            // when a tile has at least kStages steps.  Otherwise, or while incomplete, poll.
            const bool seen = landed >= 0 && KB >= kStages &&
                              __builtin_amdgcn_readfirstlane(sProbe[landed][wave]) >= wait_target;
            if (__builtin_expect(!seen, 0)) spin_until(p, wait_words + b, wait_target, lane);
            int bn = b, ntn, len, kcn;
            if (ij + 1 < my_tiles) tile_of(ij + 1, bn, ntn, len, kcn);
            iProbe = static_cast<const uint32_t*>(sgpr_ptr(wait_words + bn));
        }
        const size_t row0 = (size_t)b * BM;
        if constexpr (kRotate) ikc = kc >= 0 ? kc : __builtin_amdgcn_readfirstlane(rot_start(b, nt, le));
        iA = static_cast<const uint8_t*>(sgpr_ptr(a_base(b) + (size_t)ikc * BM * 128));
        iW = static_cast<const uint8_t*>(sgpr_ptr(w_base(le, nt) + (size_t)ikc * 256 * WRB));
        if constexpr (kLaneSmall) {
            if constexpr (kFp4) {
                const size_t nts = kGemm1 ? (size_t)(p.I >> 7) : (size_t)(p.H >> 8);
                iWsl = reinterpret_cast<const uint8_t*>(kGemm1 ? p.w1_sf : p.w2_sf) +
                       (((size_t)le * nts + nt) * KB + ikc) * 1024 + ws_tr * 4;
            }
            const float* asf = (kGemm1 ? p.pool_sf : p.l2_sf) + (size_t)b * KB * BM + sm_row;
            int blk;
            if (kGemm1) blk = lane == SA_LANES ? nt : (p.I >> 7) + nt;     // gate block, up block
            else blk = nt * 2 + (wn * WROWS) / 128;
            const float* wsf = (kGemm1 ? p.w1_sf + (size_t)le * ((2 * p.I) >> 7) * KB
                                       : p.w2_sf + (size_t)le * (p.H >> 7) * KB) + (size_t)blk * KB;
            const uint32_t* dst = p.pool_dst + row0 + sm_row;
            iSm = (sm_role == 1 ? reinterpret_cast<const uint8_t*>(wsf)
                 : sm_role == 2 ? reinterpret_cast<const uint8_t*>(dst) : reinterpret_cast<const uint8_t*>(asf)) +
                  (size_t)ikc * sm_inc;
            return;
        }
        if constexpr (kFp4) {
            // packed exponents: [E_w][n tile][K block][256 rows] words, one word = the row's four 32-value blocks
            const size_t nts = kGemm1 ? (size_t)(p.I >> 7) : (size_t)(p.H >> 8);
            iWs = static_cast<const uint8_t*>(sgpr_ptr(reinterpret_cast<const uint8_t*>(kGemm1 ? p.w1_sf : p.w2_sf) +
                                                       (((size_t)le * nts + nt) * KB + ikc) * 1024));
        }
        // (BF16: no scales; these addresses are formed but never loaded)
        iSc = static_cast<const uint8_t*>(
            sgpr_ptr((kGemm1 ? p.pool_sf : p.l2_sf) + ((size_t)b * KB + ikc) * BM));
        if constexpr (!kFp4) {
            // GEMM1: the gate block nt (the up block is I/128 blocks further); GEMM2: the wave's block
            const int blk = kGemm1 ? nt : nt * 2 + (wn * WROWS) / 128;
            iWsc = static_cast<const uint8_t*>(sgpr_ptr((kGemm1 ? p.w1_sf + (size_t)le * ((2 * p.I) >> 7) * KB
                                                                : p.w2_sf + (size_t)le * (p.H >> 7) * KB) +
                                                        (size_t)blk * KB + ikc));
        }
        if constexpr (!kGemm1) iDst = static_cast<const uint8_t*>(sgpr_ptr(p.pool_dst + row0));
    };
    set_issue_tile(-1);
    // the DMA of one K step into stage buf: straight-line code, every lane active (the probe: lane 0)
    auto issue_dma = [&](auto bufc) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
#pragma unroll
        for (int i = 0; i < A_INS; ++i) dma16(iA, a_off[i], &sA[buf][(i * NW + wave) * 1024]);
#pragma unroll
        for (int i = 0; i < B_INS; ++i) {
            if constexpr (kStreamW) dma16_nt(iW, b_off[i], &sB[buf][(i * NW + wave) * 1024]);
            else dma16(iW, b_off[i], &sB[buf][(i * NW + wave) * 1024]);
        }
        if constexpr (kLaneSmall) {
            dma4_lane(iSm, &sSmall[buf][wave * 64]);
            if constexpr (kFp4) dma4_lane(iWsl, &sWs[buf][wave * 64]);
        } else {
            if constexpr (!kBf16) {
                if (sc_lane) dma4(iSc, sm_off, &sSmall[buf][wave * 64]);
            }
            if constexpr (!kFp4 && !kBf16) {
                if (ws_lane) dma4(iWsc, sm_off, &sSmall[buf][wave * 64]);
            }
            if constexpr (!kGemm1) {
                if (tg_lane) dma4(iDst, sm_off, &sSmall[buf][wave * 64]);
            }
            if constexpr (kFp4) dma4(iWs, ws_off, &sWs[buf][wave * 64]);
        }
        if constexpr (kWait != kWaitNone) {
            if (lane == 0) dma4_coherent(iProbe, &sProbe[buf][wave]);
        }
    };
    // advance to the next step; past the last step the last step is loaded again (constant DMA count)
    auto issue_advance = [&](int landed) __attribute__((always_inline)) {
        if (ikb + 1 < KB) {
            ++ikb;
            if (!kRotate || ++ikc < KB) {
                iA += BM * 128;
                iW += 256 * WRB;
                if constexpr (kLaneSmall) {
                    iSm += sm_inc;
                    if constexpr (kFp4) iWsl += 1024;
                } else {
                    iSc += BM * 4;
                    if constexpr (!kFp4) iWsc += 4;
                    if constexpr (kFp4) iWs += 1024;
                }
            } else {                                    // wrap to K block 0
                ikc = 0;
                iA -= (size_t)(KB - 1) * BM * 128;
                iW -= (size_t)(KB - 1) * 256 * WRB;
                if constexpr (kLaneSmall) {
                    iSm -= (size_t)(KB - 1) * sm_inc;
                    if constexpr (kFp4) iWsl -= (size_t)(KB - 1) * 1024;
                } else {
                    iSc -= (size_t)(KB - 1) * BM * 4;
                    if constexpr (!kFp4) iWsc -= (size_t)(KB - 1) * 4;
                    if constexpr (kFp4) iWs -= (size_t)(KB - 1) * 1024;
                }
            }
        } else if (ij + 1 < my_tiles) {
            ikb = 0;
            ++ij;
            set_issue_tile(landed);
        }
    };

    // LDS row of this wave's weight subtile a relative to the wave's first weight row (GEMM1: the
    // first WN/2 are gate rows, the rest the matching up rows, so gate and up of one output column sit
    // in the same lane), and the lane's fragment chunk pointers
    auto wrow = [](int a) { return kGemm1 ? (a < WN / 2 ? 0 : 128) + (a % (WN / 2)) * 16 : a * 16; };
    const int xr = wm * (BM / 2) + rr;
    const int wr = (kGemm1 ? wn * HC : wn * WROWS) + rr;
    // The f8f6f4 MFMA splits an FP8 operand's K between the lane's two halves: lane group g holds
    // K 16g..16g+15 in its first 16 bytes and 64+16g..64+16g+15 in its second.  Two FP8 operands loaded
    // alike only need to agree with each other, so the FP8 path hands group g the contiguous K
    // 32g..32g+31.  An FP4 operand holds the contiguous K 32g..32g+31 in its 16 bytes (checked on the
    // chip), so against MXFP4 weights the token fragment must follow the hardware order: chunks g and
    // g + 4, which the token DMA stores where the FP8 path keeps chunks 2g and 2g + 1.  Both paths
    // therefore read the same LDS positions.
    const uint8_t* xlo = &sA[0][0] + swz(xr, 2 * g);
    const uint8_t* xhi = &sA[0][0] + swz(xr, 2 * g + 1);
    const uint8_t* wlo = &sB[0][0] + (kFp4 ? 0 : swz(wr, 2 * g));
    const uint8_t* whi = &sB[0][0] + (kFp4 ? 0 : swz(wr, 2 * g + 1));
    // MXFP4: 16 bytes per lane and fragment, chunk g of the lane's 64-byte row
    const uint8_t* wq = &sB[0][0] + wr * 64 + swz4_chunk(wr, g) * 16;

    // One K step's operands in registers: token and weight fragments, the promotion factors (token
    // scale x weight-block scale; GEMM1 has a gate and an up block) and, for GEMM2, the scatter target
    // of the wave's tokens (needed after the stage itself has been refilled).  load_head reads all but
    // the second half of the weight fragments, which load_tail reads during the step's first half.
    constexpr int NSW = kGemm1 ? 2 : 1;
    struct Frags {
        v8i x[TM];
        std::conditional_t<kFp4, v4i, v8i> w[WN];
        uint32_t ws[kFp4 ? WN : 1];   // MXFP4: UE8M0 exponent of the lane's row and K block, per fragment
        float sc[NSW][TM];
        uint32_t dst[kGemm1 ? 1 : TM];
    };
    auto load_head = [&](Frags& f, auto bufc) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
        // (MXFP4: the weight scales are applied inside the MFMA)
        const float sw0 = kFp4 || kBf16 ? 1.0f : __uint_as_float(sSmall[buf][wave * 64 + SA_LANES]);
        const float sw1 = kFp4 || kBf16 ? 1.0f : __uint_as_float(sSmall[buf][wave * 64 + SA_LANES + 1]);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int r = wm * (BM / 2) + t * 16 + rr;          // token row; loaded by wave r / SA_LANES
            const int slot = (r / SA_LANES) * 64 + r % SA_LANES;
            if constexpr (!kBf16) {
                const float sa = __uint_as_float(sSmall[buf][slot]);
                f.sc[0][t] = sa * sw0;
                if (kGemm1) f.sc[NSW - 1][t] = sa * sw1;
            }
            if (!kGemm1) f.dst[kGemm1 ? 0 : t] = sSmall[buf][slot + SA_LANES + 2];
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) f.x[t] = load_frag(xlo, xhi, buf * BM * 128 + t * 16 * 128);
#pragma unroll
        for (int a = 0; a < WN / 2; ++a) {
            if constexpr (kFp4) f.w[a] = *reinterpret_cast<const v4i*>(wq + buf * 256 * 64 + wrow(a) * 64);
            else f.w[a] = load_frag(wlo, whi, buf * 256 * 128 + wrow(a) * 128);
        }
        if constexpr (kFp4) {
#pragma unroll
            for (int a = 0; a < WN; ++a) f.ws[a] = (sWs[buf][wave * 64 + a * 16 + rr] >> (8 * g)) & 0xFFu;
        }
    };
    auto load_tail = [&](Frags& f, auto bufc) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
#pragma unroll
        for (int a = WN / 2; a < WN; ++a) {
            if constexpr (kFp4) f.w[a] = *reinterpret_cast<const v4i*>(wq + buf * 256 * 64 + wrow(a) * 64);
            else f.w[a] = load_frag(wlo, whi, buf * 256 * 128 + wrow(a) * 128);
        }
    };

    v4f acc[WN][TM];
#pragma unroll
    for (int a = 0; a < WN; ++a)
#pragma unroll
        for (int t = 0; t < TM; ++t) acc[a][t] = v4f{0.f, 0.f, 0.f, 0.f};

    int cj = 0, ckb = 0;      // compute side: tile and K step

    auto epilogue = [&](const Frags& f) __attribute__((always_inline)) {
        // lane holds acc[a][t][i]: weight row wr - rr + wrow(a) + 4g + i, token wm*BM/2 + 16t + rr
        int b, nt, le_unused, kc_unused;
        tile_of(cj, b, nt, le_unused, kc_unused);
        (void)le_unused;
        (void)kc_unused;
        const size_t row0 = (size_t)b * BM;
        if (kGemm1) {
            constexpr int HA = WN / 2;
            static_assert(HA == 2 && HC == 32 && NWN == 4, "GEMM1 epilogue store layout");
            float h[HA][TM][4];
            const int I = p.I;
            // Per-lane parts of the store addresses, laundered here so that the 64-bit addresses are
            // formed once per tile from them and wave-uniform bases, not hoisted out of the loop.
            uint32_t ln = (uint32_t)__lane_id();
            asm volatile("" : "+v"(ln));
            const uint32_t lr = ln & 15u, lg = ln >> 4;
            const uint32_t lo_go = (lr * 2u * (uint32_t)I + 4u * lg) * 4u;  // fp32 GEMM1 output (tests)
            const uint32_t lo_l2 = lr * 32u + lg * 8u;                      // L2 pool codes
            const uint32_t lo_sf = lr * 4u;                                 // L2 pool scales
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
                if (p.gemm1_out) {      // (tests) the fp32 GEMM1 output, while the accumulators live
                    char* go = reinterpret_cast<char*>(p.gemm1_out + (row0 + wm * (BM / 2) + t * 16) * (size_t)(2 * I) +
                                                       nt * 128 + wn * HC) + lo_go;
#pragma unroll
                    for (int a = 0; a < HA; ++a) {
                        *reinterpret_cast<v4f*>(go + a * 64) = acc[a][t];
                        *reinterpret_cast<v4f*>(go + (size_t)I * 4 + a * 64) = acc[a + HA][t];
                    }
                }
                if constexpr (kBf16) {
                    // BF16 x BF16: h rounded to bf16 is GEMM2's operand.  The L2 pool holds 64-value K
                    // blocks as four 16-value quarters of BM rows; this wave's 32 columns of n tile nt
                    // are K block 2nt + wn/2, quarters 2(wn&1) + a, and the lane's four columns
                    // 16a + 4g .. +3 are bytes 8g .. 8g+7 of its row's 32 (16 rows x 32 bytes = 512
                    // contiguous bytes per store instruction)
#pragma unroll
                    for (int a = 0; a < HA; ++a) {
                        const size_t q = ((size_t)b * (I >> 6) + 2 * nt + (wn >> 1)) * 4 + 2 * (wn & 1) + a;
                        *reinterpret_cast<uint2*>(p.l2_x + (q * BM + wm * (BM / 2) + t * 16) * 32 + lr * 32u + lg * 8u) =
                            uint2{bf16x2(h[a][t][0], h[a][t][1]), bf16x2(h[a][t][2], h[a][t][3])};
                    }
                    continue;
                }
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                if (g == 0) sRed[wm * (BM / 2) + t * 16 + rr][wn] = m;
            }
            if constexpr (kBf16) {
                if constexpr (kPublish) {
                    // as below: the tile's stores have completed, then one lane counts the tile
                    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
                    if (wave == 0 && lane == 0) atomicAdd(p.sched + kSchedArrival + p.max_blocks + b, 1u);
                }
#pragma unroll
                for (int a = 0; a < WN; ++a)
#pragma unroll
                    for (int t = 0; t < TM; ++t) acc[a][t] = v4f{0.f, 0.f, 0.f, 0.f};
                return;
            }
            lds_barrier();
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const int tok = wm * (BM / 2) + t * 16 + rr;
                float am = sRed[tok][0];
#pragma unroll
                for (int w = 1; w < NWN; ++w) am = fmaxf(am, sRed[tok][w]);
                const float sc = fmaxf(am, 1e-4f) / 448.0f;
                const float isc = 1.0f / sc;        // codes: h times the fp32 reciprocal of the scale
                // codes of columns 16a + 4g .. +3 of the wave's HC = 32, one dword per a
                uint32_t q[HA];
#pragma unroll
                for (int a = 0; a < HA; ++a)
                    q[a] = cvt_fp8x4(h[a][t][0] * isc, h[a][t][1] * isc, h[a][t][2] * isc, h[a][t][3] * isc);
                // (register a, lane row g) -> lane row g holds bytes 8g .. 8g+7 of the token's 32
                const auto s32 = __builtin_amdgcn_permlane32_swap(q[0], q[1], false, false);
                const auto s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
                // L2 pool: K block nt of GEMM2 is this n tile, stored as four 32-byte column quarters of
                // BM rows; this wave's quarter is wn, so its 16 tokens' 32 bytes are 512 contiguous bytes
                *reinterpret_cast<uint2*>(p.l2_x + ((size_t)b * (I >> 7) + nt) * BM * 128 + (size_t)wn * BM * 32 +
                                          (size_t)(wm * (BM / 2) + t * 16) * 32 + lo_l2) = uint2{s16[0], s16[1]};
                if (wn == 0 && g == 0)
                    *reinterpret_cast<float*>(reinterpret_cast<char*>(p.l2_sf + ((size_t)b * (I >> 7) + nt) * BM +
                                                                      wm * (BM / 2) + t * 16) + lo_sf) = sc;
            }
            if constexpr (kPublish) {
                // every wave's stores of the tile have completed (they sit in this XCD's L2); then one
                // lane counts the tile in its block's word.  sRed is free again after the barrier.
                asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
                if (wave == 0 && lane == 0) atomicAdd(p.sched + kSchedArrival + p.max_blocks + b, 1u);
            } else {
                lds_barrier();      // sRed is rewritten by the next tile
            }
        } else {
            // The wave's output: 16-token groups t, each token 64 bf16 columns (one 128-byte line of
            // its combine row).  After the MFMA, lane (rr, g) holds columns 16a + 4g .. +3 of token rr
            // for a = 0..3.  A 4x4 transpose of (register a, lane row g) gives lane (rr, g) the 32
            // contiguous bytes of subtile g; neighbour lanes rr, rr^1 then trade halves, so each store
            // writes 16 bytes per lane and eight lanes fill one token's line: two stores per group,
            // eight whole lines each.  Every lane stores (padding rows, target all ones, into the
            // spare row after the K*S*T_max combine rows), so the wave issues exactly kEpiStores
            // stores and no branch splits them.
            const uint32_t comb_rows = (uint32_t)((p.K + p.nsh) * p.S * p.T_max);
            const bool odd = rr & 1;
            const size_t col0 = (size_t)nt * 256 + wn * WROWS;
            const uint32_t byte_off = (uint32_t)g * 32 + (odd ? 16u : 0u);
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                uint32_t R[2][4];       // [h][a]: columns 16a + 4g + 2h, +1
#pragma unroll
                for (int a = 0; a < WN; ++a) {
                    R[0][a] = bf16x2(acc[a][t][0], acc[a][t][1]);
                    R[1][a] = bf16x2(acc[a][t][2], acc[a][t][3]);
                }
                transpose4_rows(R[0]);
                transpose4_rows(R[1]);
                const v4u lo = {R[0][0], R[1][0], R[0][1], R[1][1]};    // columns 16g + 0..7
                const v4u hi = {R[0][2], R[1][2], R[0][3], R[1][3]};    // columns 16g + 8..15
                const v4u recv = swap_adjacent(odd ? lo : hi);
                const uint32_t d = min(f.dst[t], comb_rows), dn = swap_adjacent(d);
                char* even_row = reinterpret_cast<char*>(p.comb + (size_t)(odd ? dn : d) * p.H + col0);
                char* odd_row = reinterpret_cast<char*>(p.comb + (size_t)(odd ? d : dn) * p.H + col0);
                *reinterpret_cast<v4u*>(even_row + byte_off) = odd ? recv : lo;
                *reinterpret_cast<v4u*>(odd_row + byte_off) = odd ? hi : recv;
            }
        }
#pragma unroll
        for (int a = 0; a < WN; ++a)
#pragma unroll
            for (int t = 0; t < TM; ++t) acc[a][t] = v4f{0.f, 0.f, 0.f, 0.f};
    };

    // Promotion of MFMA k runs kLag MFMAs after it was issued (a ring of kRing products), so the
    // VALU never waits on the matrix core; the last kLag promotions of a step run at the start of
    // the next one, with the previous step's factors.  A ring of 4 measured as fast as one of 8 and
    // leaves the registers to the per-tile bookkeeping.
    constexpr int kLag = 3, kRing = 4;
    static_assert(NMF % kRing == 0 && kLag < kRing && kLag <= NMF / 2, "promotion ring");
    v4f P[kRing];
    Frags F[2];
    auto promote = [&](const Frags& f, int k) __attribute__((always_inline)) {
        const int a = k / TM, t = k % TM;
        const int si = (kGemm1 && a >= WN / 2) ? NSW - 1 : 0;
        acc[a][t] += f.sc[si][t] * P[k % kRing];
    };
    // LDS reads of load_tail (first half) and load_head (second half), spread over the MFMAs
    constexpr int WREADS = kFp4 ? WN / 2 : WN;  // LDS reads of half the weight fragments
    constexpr int DS_TAIL = (WREADS + NMF / 2 - 1) / (NMF / 2);
    constexpr int DS_HEAD = (2 * TM + WREADS + (kFp4 ? WN : 0) + TM + 2 + (kGemm1 ? 0 : TM) + NMF / 2 - 1) / (NMF / 2);

    // One K step s on stage buf, operands in F[par] (read during step s-1).  Half-way through, after
    // the wait for stage s+1 and a barrier (every wave has finished reading stage s by then), stage
    // buf is refilled with step s+kStages and the operands of step s+1 are read into F[par ^ 1] while the
    // second half's MFMAs run.  After a tile's last step: the pending promotions, then the epilogue.
    auto step = [&](auto bufc, auto parc) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
        constexpr int par = decltype(parc)::value;
        Frags& fc = F[par];
        Frags& fn = F[par ^ 1];
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
            if (i == 0) load_tail(fc, bufc);
            if (i == NMF / 2) {
                __builtin_amdgcn_sched_barrier(0);
                // stage s+1: at most the kInFlight DMA operations of the younger stages may remain.
                // That holds whatever order stores complete in, as long as loads complete in order
                // among themselves; a tile's epilogue stores in between only add to the count.
                wait_stage_barrier<kInFlight>();
                __builtin_amdgcn_sched_barrier(0);
                issue_dma(ic<buf>{});
                load_head(fn, ic<(buf + 1) % kStages>{});
            }
            if constexpr (kBf16) {
                // unscaled operands: the two MFMAs accumulate in place, nothing to promote
                acc[i / TM][i % TM] = mfma_bf16_pair(fc.w[i / TM], fc.x[i % TM], acc[i / TM][i % TM]);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
            } else {
                if constexpr (kFp4) P[i % kRing] = mfma_fp4w(fc.w[i / TM], fc.x[i % TM], fc.ws[i / TM], v4f{0.f, 0.f, 0.f, 0.f});
                else P[i % kRing] = mfma_fp8(fc.w[i / TM], fc.x[i % TM], v4f{0.f, 0.f, 0.f, 0.f});
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                if (i >= kLag) promote(fc, i - kLag);
                else promote(fn, NMF + i - kLag);                    // previous step's last MFMAs
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // its promotion on VALU
            }
            if (i < NMF / 2) __builtin_amdgcn_sched_group_barrier(0x100, DS_TAIL, 0);      // LDS reads
            else __builtin_amdgcn_sched_group_barrier(0x100, DS_HEAD, 0);
        }
        // keep this step's promotions inside the step's block, where the schedule interleaves them
        // with the MFMAs (otherwise they may be sunk past the branches below)
#pragma unroll
        for (int a = 0; a < WN; ++a)
#pragma unroll
            for (int t = 0; t < TM; ++t) asm volatile("" : "+v"(acc[a][t]));
        issue_advance((buf + 1) % kStages);
        if (++ckb == KB) {
            if constexpr (!kBf16) {
#pragma unroll
                for (int k = NMF - kLag; k < NMF; ++k) {
                    promote(fc, k);
                    P[k % kRing] = v4f{0.f, 0.f, 0.f, 0.f};   // the next step's catch-up adds zero
                }
#pragma unroll
                for (int j = 0; j < NSW; ++j)
#pragma unroll
                    for (int t = 0; t < TM; ++t) fc.sc[j][t] = 0.f;
            }
            epilogue(fc);
            ckb = 0;
            ++cj;
        }
    };

#pragma unroll
    for (int k = 0; k < kRing; ++k) P[k] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NSW; ++j)
#pragma unroll
        for (int t = 0; t < TM; ++t) F[1].sc[j][t] = 0.f;
    issue_dma(ic<0>{});
    issue_advance(-1);
    // the other stages of the prologue
    auto prologue = [&](auto self, auto ic_j) __attribute__((always_inline)) {
        constexpr int j = decltype(ic_j)::value;
        issue_dma(ic<j>{});
        issue_advance(-1);
        if constexpr (j + 1 < kStages) self(self, ic<j + 1>{});
    };
    prologue(prologue, ic<1>{});
    wait_stage_barrier<(kStages - 1) * DMA_PER_STEP>();
    load_head(F[0], ic<0>{});
    // Steps s .. s+kUnroll-1 with their stage (I mod kStages) and operand set (I mod 2) fixed at compile
    // time; false once the last step has run.
    constexpr int kUnroll = kStages % 2 ? 2 * kStages : kStages;
    auto steps = [&](int s, auto self, auto ic_i) __attribute__((always_inline)) -> bool {
        constexpr int I = decltype(ic_i)::value;
        step(ic<I % kStages>{}, ic<I % 2>{});
        if (s + I + 1 >= nsteps) return false;
        if constexpr (I + 1 < kUnroll) return self(s, self, ic<I + 1>{});
        else return true;
    };
    for (int s = 0; s < nsteps; s += kUnroll)
        if (!steps(s, steps, ic<0>{})) break;
    wait_all_vm();      // no LDS DMA may still be landing when the phase ends
}

// expert offsets of the pool in LDS: the expert of a block is found there, so the pipeline never
// waits on a global load of its own
template <int BM, int NW, bool kFp4>
__device__ __forceinline__ void load_offsets(const Params& p) {
    auto& sOff = GemmLds<BM, NW, kFp4>::sOff();
    for (int i = threadIdx.x; i <= p.El + p.nsh; i += NW * 64) sOff[i] = p.pool_off[i];
    __syncthreads();
}

// Stream-ordered launch of one GEMM: the tiles of every pool block, spread over all work-groups.  Tiles
// map XCD-aware: work-group i runs on XCD i mod 8 and takes a run of the tile order with the other
// work-groups of that XCD.
template <int BM, int NW, bool kGemm1, bool kStreamW, bool kFp4, bool kBf16 = false>
__global__ __launch_bounds__(NW * 64, 1) void grouped_gemm_kernel(Params p) {
    const int nblocks = min((int)p.status[1], p.max_blocks);
    const int G = gridDim.x;                    // a multiple of 8
    const TilePlan plan{0, nblocks, (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3), G};
    load_offsets<BM, NW, kFp4>(p);
    gemm_phase<BM, NW, kGemm1, kStreamW, kFp4, kWaitNone, false, false, kBf16>(p, plan, nblocks);
}

// Device-wide barrier: every work-group's writes are released to memory (an L2 writeback) before it
// counts itself in *ctr, and acquired (L1 and L2 invalidated) after the count reaches the grid size.
// Needs every work-group resident at once.  The wait is bounded: past it TIMEOUT is latched and false
// returned, and the work-group then skips the rest of the launch (what follows would read routing
// results that are not complete).  The debug flag that forces waits to give up does not apply here.
__device__ __forceinline__ bool grid_barrier(const Params& p, uint32_t* ctr, int tid) {
    __shared__ int sOk;
    __syncthreads();
    if (tid < 64) {
        if (tid == 0) {
            __threadfence();
            atomicAdd(ctr, 1u);
        }
        const bool ok = spin_until<false>(p, ctr, gridDim.x, tid);
        __threadfence();
        if (tid == 0) sOk = ok;
    }
    __syncthreads();
    return sOk;
}

// Routing inside the launch, before the pull ("MoE fused operators", DeepGEMM part, 2: the expert waves
// start after the dispatch metadata, with a grid-wide sync between; "DeepGEMM Mega MoE symmetric memory
// deep analysis", 6: grid_sync).  The three routing stages run over all work-groups with the same code
// as the routing kernels (route_impl.h), each ended by a device-wide barrier; their scratch is the LDS
// of the weight stages, which the GEMM has not used yet.
template <int BM, int NW, bool kFp4>
__device__ __forceinline__ bool route_in_launch(const Params& p, int tid) {
    using Lds = GemmLds<BM, NW, kFp4>;
    int* lds = reinterpret_cast<int*>(&Lds::sB()[0][0]);
    constexpr int kLdsInts = (int)(sizeof(Lds::sB()) / sizeof(int));
    const int G = gridDim.x, wg = blockIdx.x, nthreads = NW * 64;
    const int nchunk = p.chunks * p.S;
    for (int q = wg; q < nchunk; q += G) route_count_chunk(p, q % p.chunks, q / p.chunks, lds, tid, nthreads);
    if (!grid_barrier(p, p.sched + kSchedGridBar + 0, tid)) return false;
    for (int s = wg; s < p.S; s += G) route_scan_shard(p, s, tid, nthreads);
    if (!grid_barrier(p, p.sched + kSchedGridBar + 1, tid)) return false;
    // the table: one wave per (chunk, shard), each with its own share of the LDS
    const int wave = tid >> 6, lane = tid & 63;
    constexpr int kWaveInts = kLdsInts / NW;
    const int run_ints = p.El <= 64 ? 1 : p.El, off_ints = MEGA_MOE_MAX_LOCAL_EXPERTS + 2;
    int* offs = lds + wave * kWaveInts;
    int* run = offs + off_ints;
    int* stage = run + run_ints;
    const int stage_ints = kWaveInts - off_ints - run_ints;
    for (int q = wg * NW + wave; q < nchunk; q += G * NW) {
        if (p.El <= 64) route_table_chunk<true>(p, q % p.chunks, q / p.chunks, lane, run, stage, offs, stage_ints);
        else route_table_chunk<false>(p, q % p.chunks, q / p.chunks, lane, run, stage, offs, stage_ints);
    }
    return grid_barrier(p, p.sched + kSchedGridBar + 2, tid);
}

// Launch whose work-groups hand rows over by XCD (see the top of this section): [route (kRoute),] [pull
// the pool rows (kFill),] GEMM1 [, then GEMM2 (kBoth)] over the pool blocks of the work-group's XCD.
template <int BM, int NW, bool kFill, bool kBoth, bool kStreamW, bool kFp4, bool kRoute = false, bool kBf16 = false>
__global__ __launch_bounds__(NW * 64, 1) void xcd_gemm_kernel(Params p) {
    static_assert(!kBf16 || (kBoth && !kFill && !kRoute), "BF16: both GEMMs in one launch, no pull inside it");
    const int tid = threadIdx.x, lane = tid & 63;
    if constexpr (kRoute) {
        if (!route_in_launch<BM, NW, kFp4>(p, tid)) {
            sched_exit(p, p.max_blocks, tid);      // the block count is not known: clean every block's words
            return;
        }
    }
    const int nblocks = min((int)p.status[1], p.max_blocks);
    const int W = gridDim.x / kXcds;            // work-groups per XCD (the host launches 8 W, W <= 32)
    const int x = xcc_id(), slot = blockIdx.x / kXcds;
    if (tid == 0) {
        const uint32_t bit = 1u << slot;
        const uint32_t old = x < kXcds ? atomicOr(p.sched + kSchedXcdSlots + x, bit) : bit;
        if (old & bit) atomicOr(p.status, MEGA_MOE_STATUS_PLACEMENT);
    }
    const int xs = min(x, kXcds - 1);
    const TilePlan plan{xs * nblocks / kXcds, (xs + 1) * nblocks / kXcds, slot, W};
    load_offsets<BM, NW, kFp4>(p);
    if constexpr (kFill) fill_blocks<BM>(p, plan.blo, plan.bhi, p.sched + kSchedXcdClaim + xs, lane);
    if constexpr (kBoth) {
        // Expert waves ("MoE fused operators", DeepGEMM part, 2 and 5: a wave of experts runs all its L1
        // tiles, then all its L2 tiles, and the wave is sized so its L1 tiles fill the SMs).  Here a wave
        // is a run of whole experts of the XCD's block range whose GEMM1 tiles number at least
        // p.wave_tiles (the host picks the XCD's work-group count, so every work-group has a GEMM1 tile
        // in each wave); 0 makes the whole range one wave.  The boundaries are laid out in LDS first (at
        // most kMaxWaves waves), so the loop keeps only the wave index live across the phases.
        constexpr int kMaxWaves = 64;
        __shared__ int sWave[kMaxWaves + 1];
        __shared__ int sNumWaves;
        if (tid == 0) {
            const int NT1 = p.I >> 7, range = plan.bhi - plan.blo;
            int target = p.wave_tiles > 0 ? p.wave_tiles : range * NT1;
            target = max(target, (range * NT1 + kMaxWaves - 1) / kMaxWaves);
            const auto& sOff = GemmLds<BM, NW, kFp4>::sOff();
            const int nseg = p.El + p.nsh;
            int n = 0, wb = plan.blo, i = 1;
            sWave[0] = wb;
            while (wb < plan.bhi) {
                int we = wb;
                while (we < plan.bhi && (we - wb) * NT1 < target) {
                    while (i <= nseg && sOff[i] <= we) ++i;        // the next expert boundary above we
                    we = i <= nseg ? min(sOff[i], plan.bhi) : plan.bhi;
                }
                sWave[++n] = we;
                wb = we;
            }
            sNumWaves = n;
        }
        __syncthreads();
        const int nwaves = __builtin_amdgcn_readfirstlane(sNumWaves);
        for (int w = 0; w < nwaves; ++w) {
            const TilePlan wave{__builtin_amdgcn_readfirstlane(sWave[w]), __builtin_amdgcn_readfirstlane(sWave[w + 1]),
                                slot, W};
            // The parameters are read again from the kernel-argument segment in every wave (the laundered
            // segment address keeps the loads inside the loop), so they are not held across the phases.
            auto pk = (const __attribute__((address_space(4))) Params*)__builtin_amdgcn_kernarg_segment_ptr();
            asm volatile("" : "+s"(pk));
            const Params q = *(const Params*)pk;
            gemm_phase<BM, NW, true, kStreamW, kFp4, kFill ? kWaitFill : kWaitNone, true, true, kBf16>(q, wave, nblocks);
            __syncthreads();
            gemm_phase<BM, NW, false, kStreamW, kFp4, kWaitGemm1, false, true, kBf16>(q, wave, nblocks);
            __syncthreads();
        }
    } else {
        gemm_phase<BM, NW, true, kStreamW, kFp4, kFill ? kWaitFill : kWaitNone, false, true>(p, plan, nblocks);
    }
    sched_exit(p, nblocks, tid);
}

template <int BM, bool kGemm1, bool kStreamW = false, bool kFp4 = false, bool kBf16 = false>
hipError_t launch(const Params& p, int num_cus, hipStream_t stream) {
    int grid = (num_cus + 7) / 8 * 8;
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, kWaves, kGemm1, kStreamW, kFp4, kBf16>), dim3(grid),
                       dim3(kWaves * 64), 0, stream, p);
    return hipGetLastError();
}

template <int BM, bool kFill, bool kBoth, bool kStreamW = false, bool kFp4 = false, bool kBf16 = false>
hipError_t launch_xcd(const Params& p, int num_cus, hipStream_t stream) {
    const int grid = (num_cus + 7) / 8 * 8;
    if (grid / kXcds > 32) return hipErrorInvalidConfiguration;     // one slot word per XCD
    hipLaunchKernelGGL((xcd_gemm_kernel<BM, kWaves, kFill, kBoth, kStreamW, kFp4, false, kBf16>), dim3(grid),
                       dim3(kWaves * 64), 0, stream, p);
    return hipGetLastError();
}

// Weights stream (each chunk read by one tile) when an expert is expected to fill at most one pool
// block: S*T_max*K/E routed rows per expert under uniform routing, against BLOCK_M.
bool weights_stream(const Params& p) { return (double)p.S * p.T_max * p.K / p.E <= (double)p.BM; }

}  // namespace

hipError_t launch_gemm1(const Params& p, bool fuse_fill, int num_cus, hipStream_t stream) {
    if (p.wfmt == MEGA_MOE_WEIGHTS_BF16) {
        if (fuse_fill) return hipErrorInvalidConfiguration;   // (refused by the config check)
        if (p.BM == 64)
            return weights_stream(p) ? launch<64, true, true, false, true>(p, num_cus, stream)
                                     : launch<64, true, false, false, true>(p, num_cus, stream);
        return launch<128, true, false, false, true>(p, num_cus, stream);
    }
    if (p.wfmt == MEGA_MOE_WEIGHTS_MXFP4) {
        if (p.BM == 64)
            return weights_stream(p) ? launch<64, true, true, true>(p, num_cus, stream)
                                     : launch<64, true, false, true>(p, num_cus, stream);
        return launch<128, true, false, true>(p, num_cus, stream);
    }
    if (fuse_fill)
        return p.BM == 64 ? launch_xcd<64, true, false>(p, num_cus, stream)
                          : launch_xcd<128, true, false>(p, num_cus, stream);
    if (p.BM == 64)
        return weights_stream(p) ? launch<64, true, true>(p, num_cus, stream) : launch<64, true>(p, num_cus, stream);
    return launch<128, true>(p, num_cus, stream);
}

hipError_t launch_gemm2(const Params& p, int num_cus, hipStream_t stream) {
    if (p.wfmt == MEGA_MOE_WEIGHTS_BF16) {
        if (p.BM == 64)
            return weights_stream(p) ? launch<64, false, true, false, true>(p, num_cus, stream)
                                     : launch<64, false, false, false, true>(p, num_cus, stream);
        return launch<128, false, false, false, true>(p, num_cus, stream);
    }
    if (p.wfmt == MEGA_MOE_WEIGHTS_MXFP4) {
        if (p.BM == 64)
            return weights_stream(p) ? launch<64, false, true, true>(p, num_cus, stream)
                                     : launch<64, false, false, true>(p, num_cus, stream);
        return launch<128, false, false, true>(p, num_cus, stream);
    }
    if (p.BM == 64)
        return weights_stream(p) ? launch<64, false, true>(p, num_cus, stream) : launch<64, false>(p, num_cus, stream);
    return launch<128, false>(p, num_cus, stream);
}

hipError_t launch_route_fill_gemms(const Params& p, int num_cus, hipStream_t stream) {
    // the routing's device-wide barriers need every work-group resident: one per CU, grid = CU count
    if (num_cus % kXcds || num_cus / kXcds > 32 || p.wfmt != MEGA_MOE_WEIGHTS_FP8) return hipErrorInvalidConfiguration;
    const bool sw = p.BM == 64 && weights_stream(p);
    const dim3 grid(num_cus), block(kWaves * 64);
    if (p.BM == 128)
        hipLaunchKernelGGL((xcd_gemm_kernel<128, kWaves, true, true, false, false, true>), grid, block, 0, stream, p);
    else if (sw)
        hipLaunchKernelGGL((xcd_gemm_kernel<64, kWaves, true, true, true, false, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((xcd_gemm_kernel<64, kWaves, true, true, false, false, true>), grid, block, 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_gemms(const Params& p, bool fuse_fill, int num_cus, hipStream_t stream) {
    const bool sw = p.BM == 64 && weights_stream(p);
    if (p.wfmt == MEGA_MOE_WEIGHTS_BF16) {
        if (fuse_fill) return hipErrorInvalidConfiguration;   // (refused by the config check)
        if (p.BM == 64)
            return sw ? launch_xcd<64, false, true, true, false, true>(p, num_cus, stream)
                      : launch_xcd<64, false, true, false, false, true>(p, num_cus, stream);
        return launch_xcd<128, false, true, false, false, true>(p, num_cus, stream);
    }
    if (p.wfmt == MEGA_MOE_WEIGHTS_MXFP4) {
        if (p.BM == 64)
            return sw ? launch_xcd<64, false, true, true, true>(p, num_cus, stream)
                      : launch_xcd<64, false, true, false, true>(p, num_cus, stream);
        return launch_xcd<128, false, true, false, true>(p, num_cus, stream);
    }
    if (fuse_fill)
        return p.BM == 64 ? (sw ? launch_xcd<64, true, true, true>(p, num_cus, stream)
                                : launch_xcd<64, true, true>(p, num_cus, stream))
                          : launch_xcd<128, true, true>(p, num_cus, stream);
    if (p.BM == 64)
        return sw ? launch_xcd<64, false, true, true>(p, num_cus, stream) : launch_xcd<64, false, true>(p, num_cus, stream);
    return launch_xcd<128, false, true>(p, num_cus, stream);
}

}  // namespace mm
