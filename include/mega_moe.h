/*
 * mega_moe.h -- C ABI of the fused FP8 MoE layer for one GPU's expert-parallel share (MI355X, gfx950).
 *
 * The layer (pages: "Mega-MoE kernel code walkthrough: from Dispatch to WGMMA", sections 1, 4, 6 and 9;
 * "MoE fused operators", DeepGEMM MegaMoE part) runs, on one HIP stream:
 *   1. routing metadata: per-expert send counts and a [local_expert][source_shard][slot] index table
 *      whose entries are t*K+k ("Mega-MoE notes, part 2: index table and pull", section 1);
 *   2. a round-robin pull of the routed FP8 token rows and their scales into an expert-major pool whose
 *      experts are padded to BLOCK_M rows (same page, 2.4-2.6);
 *   3. FP8 grouped GEMM gate_up, per-128-K scale promotion (same page, 5.2);
 *   4. SwiGLU and FP8 requantisation of the intermediate activation (walkthrough, section 6);
 *   5. FP8 grouped GEMM down, cast to bf16 and scattered to a per-top-k combine buffer
 *      ("DeepGEMM Mega MoE symmetric memory deep analysis", 8.1-8.2);
 *   6. the top-k weighted combine back to token-major bf16 ("Dispatch/Combine: blog theory vs DeepEP vs
 *      DeepGEMM Mega MoE", section 1; symmetric-memory page, 9.2).
 * Source ranks are emulated as S token shards that all live in this GPU's HBM; this GPU owns global experts
 * [local_rank*E_l, (local_rank+1)*E_l) (walkthrough, section 2).
 *
 * Conventions (all entry points):
 *   - Every function returns 0 on success or a negative MEGA_MOE_ERR_* code; nothing throws.
 *   - Pointers are device pointers unless the comment says host.  Device pointers must be 16-byte aligned.
 *   - Tensors are dense, row-major (C order), with the shapes given below.  The library never frees or
 *     keeps caller memory beyond the call, except the workspace, which a handle borrows until destroy.
 *   - Work is enqueued on the given stream (hipStream_t passed as void*; NULL = the null stream) and is
 *     asynchronous; inputs must stay alive and unmodified until the stream reaches the end of the call.
 *   - Conditions only the device can see (an expert id >= E, a slot past T_max) do not fail the call:
 *     the offending entry is skipped and a bit is latched in the workspace status word, which
 *     mega_moe_status reads and clears.
 */
#ifndef MEGA_MOE_H
#define MEGA_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MEGA_MOE_MAX_SHARDS 64      /* S <= 64 */
#define MEGA_MOE_MAX_TOPK 64        /* K <= 64 */
#define MEGA_MOE_MAX_EXPERTS 4096   /* E <= 4096 */
#define MEGA_MOE_MAX_LOCAL_EXPERTS 1024

/* Return codes. */
#define MEGA_MOE_OK 0
#define MEGA_MOE_ERR_INVALID_ARG (-1)          /* null / misaligned pointer, negative size, bad stage mask */
#define MEGA_MOE_ERR_UNSUPPORTED (-2)          /* a shape outside the supported set (see mega_moe_config) */
#define MEGA_MOE_ERR_TOO_MANY_TOKENS (-3)      /* tokens_per_shard[s] > max_tokens_per_shard */
#define MEGA_MOE_ERR_WORKSPACE_TOO_SMALL (-4)  /* workspace_bytes below mega_moe_workspace_bytes() */
#define MEGA_MOE_ERR_HIP (-5)                  /* a HIP runtime call failed */
#define MEGA_MOE_ERR_SCRATCH_TOO_SMALL (-6)    /* mega_moe_forward_noalloc: the config's workspace
                                                  (mega_moe_workspace_bytes) exceeds
                                                  MEGA_MOE_NOALLOC_SCRATCH_BYTES */

/* Size of the static per-GPU scratch array behind mega_moe_forward_noalloc (256 MiB). */
#define MEGA_MOE_NOALLOC_SCRATCH_BYTES (256ull << 20)

/* Device status bits (latched in the workspace, read by mega_moe_status). */
#define MEGA_MOE_STATUS_BAD_EXPERT_ID 0x1u     /* some topk_idx entry was >= E; that entry was skipped */
#define MEGA_MOE_STATUS_SLOT_OVERFLOW 0x2u     /* some (expert, shard) needed more than T_max slots */
#define MEGA_MOE_STATUS_BAD_LAYOUT 0x4u        /* a stage found workspace metadata no earlier stage wrote
                                                  (only after mega_moe_forward_stages on hand-made data);
                                                  the affected rows were skipped */
#define MEGA_MOE_STATUS_TIMEOUT 0x8u           /* FILL_IN_GEMM1 / ONE_GEMM_LAUNCH: a GEMM wave waited more
                                                  than about 2 s for pool rows or GEMM1 tiles of its block
                                                  (never expected: every counted unit is held by a running
                                                  wave); the wait was abandoned and the output is
                                                  undefined */
#define MEGA_MOE_STATUS_PLACEMENT 0x10u        /* FILL_IN_GEMM1 / ONE_GEMM_LAUNCH: two work-groups found
                                                  themselves in the same (XCD, slot), so the hardware did
                                                  not spread the launch round-robin over the eight XCDs
                                                  (never expected on MI355X); the output is undefined */

/* Config flags. */
#define MEGA_MOE_FLAG_KEEP_GEMM1_OUTPUT 0x1u   /* also store GEMM1's fp32 output [pool_rows, 2I] (tests) */
#define MEGA_MOE_FLAG_FILL_IN_GEMM1 0x2u       /* schedule of the pages ("Mega-MoE notes, part 2: index table
                                                  and pull", 2.6): GEMM1's work-groups pull the pool rows
                                                  themselves, counting each block's arrival, and a GEMM1
                                                  tile waits on its block's count instead of a kernel
                                                  boundary.  Each XCD pulls and computes its own range of
                                                  pool blocks, so the hand-over stays in its L2.  Same
                                                  results bit for bit.  FP8 weights only (the config
                                                  check refuses it with MXFP4 or BF16 weights) */
#define MEGA_MOE_FLAG_DEBUG_FORCE_TIMEOUT 0x4u /* tests: with FILL_IN_GEMM1 or ONE_GEMM_LAUNCH, every bounded
                                                  wait gives up at once and latches MEGA_MOE_STATUS_TIMEOUT
                                                  (the kernel still exits normally and zeroes its schedule
                                                  words; the output is undefined) */
#define MEGA_MOE_FLAG_DEBUG_POISON 0x8u        /* tests: before each forward, fill the pool, its scales, the
                                                  L2 pool, its scales and the combine buffer with 0xFF bytes
                                                  (NaN as e4m3fn, fp32 and bf16), so any value read before
                                                  this forward wrote it turns the output into NaN (uses
                                                  hipMemsetAsync: not for graph capture) */
#define MEGA_MOE_FLAG_DEBUG_ROUTE_LAUNCHES 0x20u /* tests: always route with the three-launch kernels, even
                                                  where the one-work-group routing (at most
                                                  S*ceil(T_max*K/64) <= 32 groups of 64 entries) or the
                                                  counts and scan in one launch (at most 8 chunks of 256
                                                  entries per shard) would be used */
#define MEGA_MOE_FLAG_ROUTE_IN_LAUNCH 0x40u    /* routing, the pull and both GEMMs in one persistent launch
                                                  (FP8 weights; all five stages selected): the routing
                                                  stages run over all work-groups, each ended by a
                                                  device-wide barrier ("DeepGEMM Mega MoE symmetric memory
                                                  deep analysis", 6: grid_sync), then the launch goes on as
                                                  with FILL_IN_GEMM1 | ONE_GEMM_LAUNCH.  Needs the whole
                                                  GPU (one work-group per CU, all resident); the waits are
                                                  bounded.  Same results bit for bit.  Timed as GEMM1 */
#define MEGA_MOE_FLAG_ONE_GEMM_LAUNCH 0x10u    /* GEMM1 and GEMM2 in one persistent launch ("MoE fused
                                                  operators", DeepGEMM part, 2: the L2 GEMM waits per m
                                                  block for its L1 n tiles): each XCD runs the GEMM1 tiles
                                                  of its range of pool blocks, counting each block's
                                                  finished n tiles, then their GEMM2 tiles, each of which
                                                  waits on its block's count.  Same results bit for bit.
                                                  With FILL_IN_GEMM1 the launch also pulls the pool rows.
                                                  Timed as GEMM1 (GEMM2 reads 0) */

/* Weight formats (mega_moe_config.weight_format). */
#define MEGA_MOE_WEIGHTS_FP8 0      /* e4m3fn codes, fp32 scales per 128x128 block                      */
#define MEGA_MOE_WEIGHTS_MXFP4 1    /* e2m1 codes, two per byte (lower K index in the low nibble), one  */
                                    /* UE8M0 exponent byte per 32 values along K: the FP8 x FP4 variant */
                                    /* of the layer ("DeepGEMM Mega MoE symmetric memory deep analysis", */
                                    /* 10.1-10.2)                                                        */
#define MEGA_MOE_WEIGHTS_BF16 2     /* BF16 x BF16: bf16 tokens and bf16 weights, no scales: the bf16    */
                                    /* kernel the pages select by operand type, whose input buffer takes */
                                    /* the tokens without scale factors ("DeepGEMM Mega MoE symmetric    */
                                    /* memory deep analysis", 5.3 and 10.1).  The pool, the L2 pool and  */
                                    /* GEMM1's output (SwiGLU rounded to bf16) hold bf16 values.  With  */
                                    /* ONE_GEMM_LAUNCH or stream-ordered kernels; FILL_IN_GEMM1 and     */
                                    /* ROUTE_IN_LAUNCH are refused (the in-launch pull is FP8's)         */

/* Stage bits for mega_moe_forward_stages.  mega_moe_forward runs all of them, in this order. */
#define MEGA_MOE_STAGE_ROUTE 0x1u     /* counts, table, pool offsets, block list, pool row metadata and */
                                      /* scatter targets, cumulative stats                              */
#define MEGA_MOE_STAGE_FILL 0x2u      /* copy of each pool row's codes and scales (needs ROUTE's      */
                                      /* outputs).  With GEMM1 also selected and FILL_IN_GEMM1 set it  */
                                      /* runs inside GEMM1's launch, timed as part of GEMM1             */
#define MEGA_MOE_STAGE_GEMM1 0x4u     /* gate_up GEMM + SwiGLU + FP8 requant into the L2 pool          */
#define MEGA_MOE_STAGE_GEMM2 0x8u     /* down GEMM, bf16, scatter to the combine buffer.  With GEMM1  */
                                      /* also selected and ONE_GEMM_LAUNCH set it runs inside GEMM1's  */
                                      /* launch, timed as part of GEMM1                                */
#define MEGA_MOE_STAGE_COMBINE 0x10u  /* top-k weighted combine into y                                 */
#define MEGA_MOE_STAGE_ALL 0x1Fu
#define MEGA_MOE_NUM_STAGES 5

typedef struct mega_moe_config {
    int32_t num_shards;           /* S: emulated source ranks, 1..64                                   */
    int32_t max_tokens_per_shard; /* T_max: capacity per shard, >= 1                                    */
    int32_t hidden;               /* H: multiple of 256, 256..16384                                     */
    int32_t intermediate;         /* I: multiple of 128, 128..16384                                     */
    int32_t num_experts;          /* E: global experts, 1..4096, a multiple of num_local_experts        */
    int32_t num_local_experts;    /* E_l: experts owned by this GPU, 1..1024                            */
    int32_t local_rank;           /* r: owns experts [r*E_l, (r+1)*E_l); 0 <= r < E/E_l                 */
    int32_t topk;                 /* K: 1..64                                                           */
    int32_t block_m;              /* BLOCK_M of the pool: 64 or 128; 0 picks from the expected rows     */
    uint32_t flags;               /* MEGA_MOE_FLAG_*                                                    */
    int32_t num_shared_experts;   /* 0 or 1.  1: a shared expert (intermediate size I, weights stored   */
                                  /* as expert E_l of W1/W2) runs on every valid token of this rank's   */
                                  /* own shard, shard local_rank (needs local_rank < S and K < 64), and */
                                  /* its output is added with weight 1 after the routed slots           */
                                  /* ("DeepGEMM Mega MoE symmetric memory deep analysis", 4.1, 8.1-8.2, */
                                  /* 9.2: the shared expert reads the rank's own input buffer and        */
                                  /* writes the extra combine slot K locally)                           */
    int32_t weight_format;        /* MEGA_MOE_WEIGHTS_FP8 (default), _MXFP4 or _BF16                   */
} mega_moe_config;

/* Byte offsets of the regions inside the workspace (for tests and tools) plus the resolved sizes. */
typedef struct mega_moe_layout {
    int32_t block_m;          /* resolved BLOCK_M                                                 */
    int32_t route_chunks;     /* routing chunks per shard                                         */
    int32_t max_pool_blocks;  /* capacity in BLOCK_M blocks: ceil(S*T_max*min(K,E_l)/BM) + E_l     */
                              /*   (+ ceil(T_max/BM) with a shared expert)                          */
    int32_t reserved;
    uint64_t status;          /* uint32 [0]: status bits; uint32 [1]: number of pool blocks (last forward) */
    uint64_t chunk_hist;      /* int32 [S][chunks][E]                                             */
    uint64_t chunk_base;      /* int32 [S][chunks][E_l]                                           */
    uint64_t send;            /* int32 [S][E]: pairs of shard s routed to global expert e         */
    uint64_t recv;            /* int32 [E_l][S]: recv[le][s] = send[s][r*E_l+le]                  */
    uint64_t recv_tot;        /* int32 [E_l]                                                      */
    uint64_t pool_off;        /* int32 [E_l+2]: first pool block of each local expert; [E_l] ends */
                              /*   the routed segments, [E_l+1] the shared expert's segment (the    */
                              /*   own shard's valid tokens in order; equal to [E_l] without one)  */
    uint64_t block_expert;    /* int32 [max_pool_blocks]: local expert of each pool block          */
    uint64_t block_index;     /* int32 [max_pool_blocks]: m-block index inside its expert          */
    uint64_t table;           /* int32 [E_l][S][T_max]: t*K+k, slots >= recv[le][s] unspecified    */
    uint64_t pool_x;          /* uint8 [max_pool_blocks][H/128][BM][128] e4m3fn: pool row b*BM+m,  */
                              /*   columns kb*128..+127 at ((b*(H/128) + kb)*BM + m)*128 (tiled, so */
                              /*   one block's K step is one contiguous 16 KB chunk at BM = 128)     */
                              /*   BF16: the same tiling of 2H bytes per row, [H/64] chunks of 64     */
                              /*   bf16 values                                                       */
    uint64_t pool_sf;         /* float [max_pool_blocks][H/128][BM]: block-major, so the BM scales */
                              /*   of one block and K block are contiguous (empty with BF16)         */
    uint64_t pool_meta;       /* uint32 [max_pool_blocks*BM][3] = {shard, token, k}; padding = ~0  */
    uint64_t pool_dst;        /* uint32 [max_pool_blocks*BM]: comb row k*S*T_max + shard*T_max +   */
                              /*   token of the pool row (the GEMM2 scatter target); padding = ~0  */
    uint64_t l2_x;            /* uint8 [max_pool_blocks][I/128][4][BM][32] e4m3fn: per block and K  */
                              /* block, four 32-column quarters of BM rows.  BF16: bf16            */
                              /* [max_pool_blocks][I/64][4][BM][16], the same 128-byte K blocks    */
    uint64_t l2_sf;           /* float [max_pool_blocks][I/128][BM], block-major like pool_sf      */
                              /*   (empty with BF16)                                                 */
    uint64_t comb;            /* bf16 [K + n_shared][S*T_max][H]: rows of routed (k, shard, token) */
                              /* (plane K: the shared expert's rows of the own shard), then one    */
                              /* spare row that takes GEMM2's padding rows                        */
    uint64_t gemm1_out;       /* float [max_pool_blocks*BM][2I] if MEGA_MOE_FLAG_KEEP_GEMM1_OUTPUT  */
    uint64_t sched;           /* uint32 [64 + 2*max_pool_blocks]: schedule words of FILL_IN_GEMM1 / */
                              /*   ONE_GEMM_LAUNCH: [2] exit ticket, [8 + x] next fill unit of XCD  */
                              /*   x, [16 + x] slots of XCD x taken, [64 + b] fill units of pool    */
                              /*   block b done, [64 + max_pool_blocks + b] GEMM1 n tiles of block  */
                              /*   b done; all zero between forwards                               */
    uint64_t total;           /* bytes needed                                                     */
} mega_moe_layout;

typedef struct mega_moe_handle mega_moe_handle;

/* Bytes of device workspace the config needs (host-only arithmetic; no GPU call).  The pages' extension
 * is asked the same way for the size of its buffer before the caller allocates it and hands it over
 * ("DeepGEMM Mega MoE symmetric memory deep analysis", 5.1 and 10.1).
 * Errors: INVALID_ARG (null pointer), UNSUPPORTED (config outside the limits above). */
int32_t mega_moe_workspace_bytes(const mega_moe_config* cfg, uint64_t* bytes_out /* host */);

/* Create a handle over a caller-allocated workspace (the size query then caller allocation follows the
 * pages' buffer setup: "DeepGEMM Mega MoE symmetric memory deep analysis", 5.1).  Zeroes the workspace on
 * `stream`.  The workspace belongs to this handle until mega_moe_destroy; one handle must not run two
 * forwards concurrently.  The current HIP device at init is the device the handle runs on.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP. */
int32_t mega_moe_init(const mega_moe_config* cfg, void* workspace, uint64_t workspace_bytes, void* stream,
                      mega_moe_handle** out /* host */);

/* One-time weight transform (the pages' kernels take their weights in a transformed layout too:
 * "DeepGEMM Mega MoE symmetric memory deep analysis", 10.2).  Copies W1 and W2 into the tiled order the
 * grouped GEMMs stream, where one K step of one n tile is one contiguous 32 KB chunk:
 * E_w = E_l + num_shared_experts experts are packed (the shared expert last).
 *   w1_packed  uint8 [E_w][I/128][H/128][256][128]: chunk (le, nt, kb), row r, byte j holds
 *              W1[le][r < 128 ? nt*128 + r : I + nt*128 + r - 128][kb*128 + j]   (128 gate rows, then
 *              the matching 128 up rows)
 *   w2_packed  uint8 [E_w][H/256][I/128][256][128]: chunk (le, nt, kb), row r, byte j holds
 *              W2[le][nt*256 + r][kb*128 + j]
 * w1 / w2 are the row-major [E_w][2I][H] / [E_w][H][I] e4m3fn tensors below; the packed buffers have the
 * same byte counts and must not overlap them.
 * With weight_format MEGA_MOE_WEIGHTS_MXFP4 the inputs are the e2m1 codes, uint8 [E_w][2I][H/2] and
 * [E_w][H][I/2], and each packed row holds 64 bytes per K step: w1_packed [E_w][I/128][H/128][256][64],
 * w2_packed [E_w][H/256][I/128][256][64], same row order.
 * With weight_format MEGA_MOE_WEIGHTS_BF16 the inputs are bf16 [E_w][2I][H] and [E_w][H][I], packed as
 * bytes with 128-byte (64-value) K chunks: w1_packed [E_w][I/128][H/64][256][128] (chunk (le, nt, kb), row
 * r, bytes of W1 values kb*64 .. kb*64+63), w2_packed [E_w][H/256][I/64][256][128].
 * Asynchronous on `stream`; no handle is needed.
 * Errors: INVALID_ARG (null or not 16-byte aligned pointer), UNSUPPORTED (config), HIP. */
int32_t mega_moe_pack_weights(const mega_moe_config* cfg, const void* w1, const void* w2, void* w1_packed,
                              void* w2_packed, void* stream);

/* One-time transform of MXFP4 weight exponents (weight_format MEGA_MOE_WEIGHTS_MXFP4 only).  The pages
 * pass the FP4 kernel's scale factors packed along K and transposed for the kernel ("DeepGEMM Mega MoE
 * symmetric memory deep analysis", 10.1-10.2); here they follow the packed weights' chunks, so one GEMM
 * step reads a chunk's exponents as 1 KB of consecutive words:
 *   w1_sf          uint8 [E_w][2I][H/32]: UE8M0 exponent of W1[le][n][32j .. 32j+31] at [le][n][j]
 *   w2_sf          uint8 [E_w][H][I/32]
 *   w1_sf_packed   uint8 [E_w][I/128][H/128][256][4]: chunk (le, nt, kb), row r, byte j holds
 *                  w1_sf[le][r < 128 ? nt*128 + r : I + nt*128 + r - 128][4*kb + j]
 *   w2_sf_packed   uint8 [E_w][H/256][I/128][256][4]: byte j of (le, nt, kb, r) holds w2_sf[le][nt*256 + r][4*kb + j]
 * The packed buffers have the same byte counts as the inputs and must not overlap them.  Asynchronous on
 * `stream`; no handle is needed.
 * Errors: INVALID_ARG (null or not 4-byte aligned pointer, or an FP8 config), UNSUPPORTED (config), HIP. */
int32_t mega_moe_pack_scales(const mega_moe_config* cfg, const void* w1_sf, const void* w2_sf, void* w1_sf_packed,
                             void* w2_sf_packed, void* stream);

/* The whole layer.  Shapes (S, T_max, H, I, E_l, K from the config):
 *   tokens_per_shard  host int32 [S], each in 0..T_max: valid tokens of each shard (rows t >= T_s are
 *                     neither read nor written)
 *   x                 uint8 [S][T_max][H], e4m3fn codes
 *   x_sf              float [S][T_max][H/128], per-token per-128-column scales
 *   topk_idx          int64 [S][T_max][K], global expert ids; < 0 means "no expert"
 *   topk_weights      float [S][T_max][K]
 *   w1                W1 packed by mega_moe_pack_weights from uint8 [E_w][2I][H] e4m3fn (rows 0..I-1
 *                     gate, I..2I-1 up; E_w = E_l + num_shared_experts, the shared expert last)
 *   w1_sf             float [E_w][2I/128][H/128], 128x128 block scales of the unpacked W1
 *   w2                W2 packed by mega_moe_pack_weights from uint8 [E_w][H][I] e4m3fn
 *   w2_sf             float [E_w][H/128][I/128]
 *                     With weight_format MEGA_MOE_WEIGHTS_MXFP4: w1 / w2 are the packed e2m1 codes and
 *                     w1_sf / w2_sf the exponents packed by mega_moe_pack_scales (uint8, passed through
 *                     the same float pointers)
 *                     With weight_format MEGA_MOE_WEIGHTS_BF16: x is bf16 [S][T_max][H], w1 / w2 are packed
 *                     from bf16 weights, and x_sf, w1_sf, w2_sf are not read (NULL allowed)
 *   y                 bf16 [S][T_max][H] output: y[s,t] = sum over k with a local expert of
 *                     w[s,t,k] * Expert(x[s,t]), plus Shared(x[s,t]) for s = local_rank when the
 *                     config has a shared expert; a token with nothing to add gets a zero row
 *   cum_recv_stats    int32 [E_l] or NULL: cum_recv_stats[le] += rows received by local expert le
 *                     (the caller resets it; "DeepGEMM Mega MoE symmetric memory deep analysis", 10.1)
 * Errors: INVALID_ARG, TOO_MANY_TOKENS, HIP.  Leaves the workspace ready for the next call. */
int32_t mega_moe_forward(mega_moe_handle* h, const int32_t* tokens_per_shard, const void* x, const float* x_sf,
                         const int64_t* topk_idx, const float* topk_weights, const void* w1, const float* w1_sf,
                         const void* w2, const float* w2_sf, void* y, int32_t* cum_recv_stats, void* stream);

/* As mega_moe_forward, running only the stages in `stages` (MEGA_MOE_STAGE_* bits).  A stage reads what
 * the earlier stages left in the workspace, so tests can place their own intermediate data there
 * (see mega_moe_query_layout) and run one stage on it.  Pointers a selected stage does not read may
 * be NULL.  Errors: as mega_moe_forward; INVALID_ARG for stages == 0 or unknown bits. */
int32_t mega_moe_forward_stages(mega_moe_handle* h, uint32_t stages, const int32_t* tokens_per_shard,
                                const void* x, const float* x_sf, const int64_t* topk_idx,
                                const float* topk_weights, const void* w1, const float* w1_sf, const void* w2,
                                const float* w2_sf, void* y, int32_t* cum_recv_stats, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the whole layer as mega_moe_forward, with no handle and no allocation.
 * Its workspace is a static device array of MEGA_MOE_NOALLOC_SCRATCH_BYTES (256 MiB) that every GPU the
 * library runs on holds from the library's first use there until the process ends; the caller passes
 * only inputs and outputs (the same ones as mega_moe_forward, weights packed by mega_moe_pack_weights)
 * and the config.  The forward zeroes the status word and schedule words on `stream` with a kernel (no
 * memset), so the call may be captured into a HIP graph.
 *   device_status  uint32 (device) or NULL: receives the forward's MEGA_MOE_STATUS_* bits.
 * Every call on one GPU uses that GPU's one array: calls that overlap on a GPU (two streams, two host
 * threads) race, and must be serialised by the caller.  The array keeps the last call's contents.
 * Errors: INVALID_ARG, UNSUPPORTED (config, or the DEBUG_POISON / KEEP_GEMM1_OUTPUT flags), TOO_MANY_TOKENS,
 * SCRATCH_TOO_SMALL (mega_moe_workspace_bytes(cfg) > MEGA_MOE_NOALLOC_SCRATCH_BYTES), HIP. */
int32_t mega_moe_forward_noalloc(const mega_moe_config* cfg, const int32_t* tokens_per_shard /* host, [S] */,
                                 const void* x, const float* x_sf, const int64_t* topk_idx,
                                 const float* topk_weights, const void* w1, const float* w1_sf, const void* w2,
                                 const float* w2_sf, void* y, int32_t* cum_recv_stats, uint32_t* device_status,
                                 void* stream);

/* Region offsets of the handle's workspace (this library's own call, for tests and tools that read or
 * place intermediate data; the pages have no counterpart).  Errors: INVALID_ARG. */
int32_t mega_moe_query_layout(const mega_moe_handle* h, mega_moe_layout* out /* host */);

/* Synchronise `stream`, read and clear the device status word into *device_flags (host).  This library's
 * own call (the pages define no status readback): conditions only the device sees (MEGA_MOE_STATUS_*)
 * are latched in the workspace and read here.  Errors: INVALID_ARG, HIP. */
int32_t mega_moe_status(mega_moe_handle* h, void* stream, uint32_t* device_flags /* host */);

/* Per-stage timing.  mega_moe_set_timing(h, 1) starts (and resets) accumulation: every later forward
 * records HIP events around each stage on its own stream, without synchronising.  mega_moe_stage_times
 * waits for the recorded events and writes, per stage, the mean milliseconds over the forwards timed
 * since the reset (MEGA_MOE_NUM_STAGES floats to ms; 0 for a stage that never ran) and the number of
 * timed forwards to *count (host, may be NULL).  mega_moe_set_timing(h, 0) stops recording.
 * Errors: INVALID_ARG, HIP. */
int32_t mega_moe_set_timing(mega_moe_handle* h, int32_t enable);
int32_t mega_moe_stage_times(mega_moe_handle* h, float* ms /* host, MEGA_MOE_NUM_STAGES */,
                             int32_t* count /* host, nullable */);

/* Release the handle (not the workspace).  Accepts NULL. */
void mega_moe_destroy(mega_moe_handle* h);

/* Static text for a return code. */
const char* mega_moe_strerror(int32_t code);

#ifdef __cplusplus
}
#endif
#endif /* MEGA_MOE_H */
