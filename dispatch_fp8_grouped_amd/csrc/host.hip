// Host side of libmegamoe: argument checks, workspace layout, stage launches, status and timing.
//
// The setup mirrors the pages' buffer handling ("DeepGEMM Mega MoE symmetric memory deep analysis",
// 4.1-4.2 and 5.1): the caller asks for a size, allocates one block of device memory and hands it
// over; the library carves it into fixed regions.  Pool capacity follows the same page's bound
// (4.2): ceil(max routed rows / BLOCK_M) + E_l blocks.  There is no cross-GPU symmetric memory here:
// the S source shards live in this GPU's HBM, so every pointer is local.
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "mm_internal.h"

using mm::Params;

static constexpr int kTimingSets = 64;

struct mega_moe_handle {
    mega_moe_config cfg;
    mega_moe_layout lay;
    uint8_t* ws;
    uint64_t ws_bytes;
    int device;
    int num_cus;
    // stage timing: a ring of event sets, folded into running sums when a set is reused
    bool timing;
    int next_set;                                   // forwards recorded since the reset
    hipEvent_t ev[kTimingSets][MEGA_MOE_NUM_STAGES + 1];
    uint32_t ran[kTimingSets];
    bool pending[kTimingSets];
    double sum_ms[MEGA_MOE_NUM_STAGES];
    int runs[MEGA_MOE_NUM_STAGES];
};

namespace {

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int32_t check_config(const mega_moe_config* c) {
    if (!c) return MEGA_MOE_ERR_INVALID_ARG;
    if (c->num_shards < 1 || c->num_shards > MEGA_MOE_MAX_SHARDS) return MEGA_MOE_ERR_UNSUPPORTED;
    if (c->max_tokens_per_shard < 1) return MEGA_MOE_ERR_UNSUPPORTED;
    if (c->hidden < 256 || c->hidden > 16384 || c->hidden % 256 != 0) return MEGA_MOE_ERR_UNSUPPORTED;
    if (c->intermediate < 128 || c->intermediate > 16384 || c->intermediate % 128 != 0)
        return MEGA_MOE_ERR_UNSUPPORTED;
    if (c->num_local_experts < 1 || c->num_local_experts > MEGA_MOE_MAX_LOCAL_EXPERTS)
        return MEGA_MOE_ERR_UNSUPPORTED;
    if (c->num_experts < 1 || c->num_experts > MEGA_MOE_MAX_EXPERTS ||
        c->num_experts % c->num_local_experts != 0)
        return MEGA_MOE_ERR_UNSUPPORTED;
    if (c->local_rank < 0 || c->local_rank >= c->num_experts / c->num_local_experts)
        return MEGA_MOE_ERR_UNSUPPORTED;
    if (c->topk < 1 || c->topk > MEGA_MOE_MAX_TOPK) return MEGA_MOE_ERR_UNSUPPORTED;
    if (c->block_m != 0 && c->block_m != 64 && c->block_m != 128) return MEGA_MOE_ERR_UNSUPPORTED;
    if (c->flags & ~(MEGA_MOE_FLAG_KEEP_GEMM1_OUTPUT | MEGA_MOE_FLAG_FILL_IN_GEMM1 |
                     MEGA_MOE_FLAG_DEBUG_FORCE_TIMEOUT | MEGA_MOE_FLAG_DEBUG_POISON |
                     MEGA_MOE_FLAG_ONE_GEMM_LAUNCH | MEGA_MOE_FLAG_DEBUG_ROUTE_LAUNCHES |
                     MEGA_MOE_FLAG_ROUTE_IN_LAUNCH))
        return MEGA_MOE_ERR_UNSUPPORTED;
    // table entries are int32 t*K+k
    if ((int64_t)c->max_tokens_per_shard * c->topk >= (int64_t)1 << 31) return MEGA_MOE_ERR_UNSUPPORTED;
    // the shared expert reads the own shard and takes combine slot K (a lane of the combine's ballot)
    if (c->num_shared_experts < 0 || c->num_shared_experts > 1) return MEGA_MOE_ERR_UNSUPPORTED;
    if (c->num_shared_experts && (c->local_rank >= c->num_shards || c->topk >= 64)) return MEGA_MOE_ERR_UNSUPPORTED;
    if (c->weight_format != MEGA_MOE_WEIGHTS_FP8 && c->weight_format != MEGA_MOE_WEIGHTS_MXFP4 &&
        c->weight_format != MEGA_MOE_WEIGHTS_BF16)
        return MEGA_MOE_ERR_UNSUPPORTED;
    // BF16 x BF16: stream-ordered kernels, or both GEMMs in one launch (no pull inside it)
    if (c->weight_format == MEGA_MOE_WEIGHTS_BF16 &&
        (c->flags & (MEGA_MOE_FLAG_FILL_IN_GEMM1 | MEGA_MOE_FLAG_ROUTE_IN_LAUNCH)))
        return MEGA_MOE_ERR_UNSUPPORTED;
    // the arrival-counted fill (and the launch that also routes) is built for FP8 weights only
    if (c->weight_format == MEGA_MOE_WEIGHTS_MXFP4 &&
        (c->flags & (MEGA_MOE_FLAG_FILL_IN_GEMM1 | MEGA_MOE_FLAG_ROUTE_IN_LAUNCH)))
        return MEGA_MOE_ERR_UNSUPPORTED;
    // pool rows and combine rows (K*S*T_max) are int32 / uint32 indices in the kernels
    if ((int64_t)c->num_shards * c->max_tokens_per_shard * (c->topk + 1) + (int64_t)c->num_local_experts * 128 +
            (int64_t)c->max_tokens_per_shard + 128 >=
        (int64_t)1 << 31)
        return MEGA_MOE_ERR_UNSUPPORTED;
    return MEGA_MOE_OK;
}

int resolve_block_m(const mega_moe_config* c) {
    if (c->block_m) return c->block_m;
    // expected rows per local expert under uniform routing: S*T_max*K/E
    const double rows = (double)c->num_shards * c->max_tokens_per_shard * c->topk / c->num_experts;
    return rows <= 64.0 ? 64 : 128;
}

void make_layout(const mega_moe_config* c, mega_moe_layout* L) {
    memset(L, 0, sizeof(*L));
    const uint64_t S = c->num_shards, T = c->max_tokens_per_shard, H = c->hidden, I = c->intermediate;
    const uint64_t E = c->num_experts, El = c->num_local_experts, K = c->topk;
    const int bm = resolve_block_m(c);
    const uint64_t chunks = (T * K + mm::kRouteChunk - 1) / mm::kRouteChunk;
    const uint64_t kloc = K < El ? K : El;
    const uint64_t max_routed = S * T * kloc;
    const uint64_t nsh = (uint64_t)c->num_shared_experts;
    const uint64_t max_blocks = (max_routed + bm - 1) / bm + El + nsh * ((T + bm - 1) / bm);
    const uint64_t rows = max_blocks * bm;
    L->block_m = bm;
    L->route_chunks = (int32_t)chunks;
    L->max_pool_blocks = (int32_t)max_blocks;
    uint64_t o = 0;
    auto take = [&](uint64_t bytes) { const uint64_t at = o; o = align_up(o + bytes); return at; };
    L->status = take(kAlign);
    L->chunk_hist = take(S * chunks * E * 4);
    L->chunk_base = take(S * chunks * El * 4);
    L->send = take(S * E * 4);
    L->recv = take(El * S * 4);
    L->recv_tot = take(El * 4);
    L->pool_off = take((El + 2) * 4);
    L->block_expert = take(max_blocks * 4);
    L->block_index = take(max_blocks * 4);
    L->table = take(El * S * T * 4);
    // BF16 x BF16: pool and L2 pool hold bf16 values (two bytes each) and no scales
    const bool bf16 = c->weight_format == MEGA_MOE_WEIGHTS_BF16;
    const uint64_t eb = bf16 ? 2 : 1;
    L->pool_x = take(rows * H * eb);
    L->pool_sf = take(bf16 ? 0 : rows * (H / 128) * 4);
    L->pool_meta = take(rows * 3 * 4);
    L->pool_dst = take(rows * 4);
    L->l2_x = take(rows * I * eb);
    L->l2_sf = take(bf16 ? 0 : rows * (I / 128) * 4);
    L->comb = take(((K + nsh) * S * T + 1) * H * 2);   // + one spare row: GEMM2 stores padding rows there
    L->gemm1_out = (c->flags & MEGA_MOE_FLAG_KEEP_GEMM1_OUTPUT) ? take(rows * 2 * I * 4) : 0;
    L->sched = take((mm::kSchedArrival + 2 * max_blocks) * 4);
    L->total = o;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Wait for event set k and add its stage times to the running sums.
int32_t fold_times(mega_moe_handle* h, int k) {
    if (hipEventSynchronize(h->ev[k][MEGA_MOE_NUM_STAGES]) != hipSuccess) return MEGA_MOE_ERR_HIP;
    for (int i = 0; i < MEGA_MOE_NUM_STAGES; ++i) {
        if (!(h->ran[k] & (1u << i))) continue;
        float t = 0.f;
        if (hipEventElapsedTime(&t, h->ev[k][i], h->ev[k][i + 1]) != hipSuccess) return MEGA_MOE_ERR_HIP;
        h->sum_ms[i] += t;
        h->runs[i] += 1;
    }
    h->pending[k] = false;
    return MEGA_MOE_OK;
}


// Caller pointers of one forward.
struct ForwardArgs {
    const int32_t* tps;
    const void* x;
    const float* x_sf;
    const int64_t* topk_idx;
    const float* topk_weights;
    const void* w1;
    const float* w1_sf;
    const void* w2;
    const float* w2_sf;
    void* y;
    int32_t* cum;
};

// The selected stages of one forward over the workspace `w` (layout L) on the current device.  `h`
// (nullable) supplies the stage-timing events.
int32_t run_forward(const mega_moe_config& c, const mega_moe_layout& L, uint8_t* w, int num_cus, uint32_t stages,
                    const ForwardArgs& a, hipStream_t st, mega_moe_handle* h) {
    if (!a.tps) return MEGA_MOE_ERR_INVALID_ARG;
    if (stages == 0 || (stages & ~MEGA_MOE_STAGE_ALL)) return MEGA_MOE_ERR_INVALID_ARG;
    const bool route = stages & MEGA_MOE_STAGE_ROUTE, fill = stages & MEGA_MOE_STAGE_FILL;
    const bool g1 = stages & MEGA_MOE_STAGE_GEMM1, g2 = stages & MEGA_MOE_STAGE_GEMM2;
    const bool comb = stages & MEGA_MOE_STAGE_COMBINE;
    // pointers each selected stage reads or writes
    auto need = [](bool used, const void* ptr) { return !used || (ptr && aligned16(ptr)); };
    const bool scaled = c.weight_format != MEGA_MOE_WEIGHTS_BF16;     // BF16 x BF16 takes no scales
    if (!need(route || comb, a.topk_idx) || !need(fill, a.x) || !need(fill && scaled, a.x_sf) ||
        !need(g1, a.w1) || !need(g1 && scaled, a.w1_sf) || !need(g2, a.w2) || !need(g2 && scaled, a.w2_sf) ||
        !need(comb, a.topk_weights) || !need(comb, a.y))
        return MEGA_MOE_ERR_INVALID_ARG;
    if (a.cum && ((uintptr_t)a.cum & 3u)) return MEGA_MOE_ERR_INVALID_ARG;

    Params p;
    memset(&p, 0, sizeof(p));
    p.S = c.num_shards;
    p.T_max = c.max_tokens_per_shard;
    p.H = c.hidden;
    p.I = c.intermediate;
    p.E = c.num_experts;
    p.El = c.num_local_experts;
    p.nsh = c.num_shared_experts;
    p.own = c.local_rank;
    p.wfmt = c.weight_format;
    p.lo = c.local_rank * c.num_local_experts;
    p.K = c.topk;
    p.BM = L.block_m;
    p.chunks = L.route_chunks;
    p.max_blocks = L.max_pool_blocks;
    // one-launch GEMMs: an expert wave holds at least one GEMM1 tile per work-group of an XCD
    p.wave_tiles = ((num_cus + 7) / 8 * 8) / 8;
    p.flags = c.flags;
    for (int s = 0; s < c.num_shards; ++s) {
        const int32_t t = a.tps[s];
        if (t < 0) return MEGA_MOE_ERR_INVALID_ARG;
        if (t > c.max_tokens_per_shard) return MEGA_MOE_ERR_TOO_MANY_TOKENS;
        p.tps[s] = t;
    }
    p.status = reinterpret_cast<uint32_t*>(w + L.status);
    p.chunk_hist = reinterpret_cast<int*>(w + L.chunk_hist);
    p.chunk_base = reinterpret_cast<int*>(w + L.chunk_base);
    p.send = reinterpret_cast<int*>(w + L.send);
    p.recv = reinterpret_cast<int*>(w + L.recv);
    p.recv_tot = reinterpret_cast<int*>(w + L.recv_tot);
    p.pool_off = reinterpret_cast<int*>(w + L.pool_off);
    p.block_expert = reinterpret_cast<int*>(w + L.block_expert);
    p.block_index = reinterpret_cast<int*>(w + L.block_index);
    p.table = reinterpret_cast<int*>(w + L.table);
    p.pool_x = w + L.pool_x;
    p.pool_sf = reinterpret_cast<float*>(w + L.pool_sf);
    p.pool_meta = reinterpret_cast<uint32_t*>(w + L.pool_meta);
    p.pool_dst = reinterpret_cast<uint32_t*>(w + L.pool_dst);
    p.l2_x = w + L.l2_x;
    p.l2_sf = reinterpret_cast<float*>(w + L.l2_sf);
    p.comb = reinterpret_cast<uint16_t*>(w + L.comb);
    p.gemm1_out = L.gemm1_out ? reinterpret_cast<float*>(w + L.gemm1_out) : nullptr;
    p.sched = reinterpret_cast<uint32_t*>(w + L.sched);
    p.x = static_cast<const uint8_t*>(a.x);
    p.x_sf = a.x_sf;
    p.topk_idx = a.topk_idx;
    p.topk_w = a.topk_weights;
    p.w1 = static_cast<const uint8_t*>(a.w1);
    p.w1_sf = a.w1_sf;
    p.w2 = static_cast<const uint8_t*>(a.w2);
    p.w2_sf = a.w2_sf;
    p.y = static_cast<uint16_t*>(a.y);
    p.cum = a.cum;

    int32_t rc = MEGA_MOE_OK;
    // with FILL_IN_GEMM1 (and both stages selected) the fill runs inside GEMM1's launch; with
    // ONE_GEMM_LAUNCH (and both GEMMs selected) GEMM2 runs inside it too
    const bool fused_fill = fill && g1 && (c.flags & MEGA_MOE_FLAG_FILL_IN_GEMM1);
    const bool one_launch = g1 && g2 && (c.flags & MEGA_MOE_FLAG_ONE_GEMM_LAUNCH);
    // with ROUTE_IN_LAUNCH (and routing, fill and both GEMMs selected) all four run in GEMM1's launch
    const bool all_in_one = route && fill && g1 && g2 && (c.flags & MEGA_MOE_FLAG_ROUTE_IN_LAUNCH);
    const bool on[MEGA_MOE_NUM_STAGES] = {route && !all_in_one, fill && !fused_fill && !all_in_one, g1,
                                          g2 && !one_launch && !all_in_one, comb};
    const bool timing = h && h->timing;
    const int set = h ? h->next_set % kTimingSets : 0;
    if (timing && h->pending[set] && fold_times(h, set) != MEGA_MOE_OK) rc = MEGA_MOE_ERR_HIP;
    uint32_t ran_mask = 0;
    auto mark = [&](int i) {
        if (timing && !rc && hipEventRecord(h->ev[set][i], st) != hipSuccess) rc = MEGA_MOE_ERR_HIP;
    };
    if (!rc && route && (c.flags & MEGA_MOE_FLAG_DEBUG_POISON)) {
        // every region a stage fills for a later one: a read of anything this forward did not write
        // shows up as NaN in the output.  The fills are memsets, which a captured HIP graph must not
        // hold: refused on a capturing stream.
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) != hipSuccess) rc = MEGA_MOE_ERR_HIP;
        else if (cs != hipStreamCaptureStatusNone) rc = MEGA_MOE_ERR_UNSUPPORTED;
        const uint64_t regions[][2] = {{L.pool_x, L.pool_sf}, {L.pool_sf, L.pool_meta}, {L.l2_x, L.l2_sf},
                                       {L.l2_sf, L.comb}};
        for (const auto& r : regions)
            if (!rc && hipMemsetAsync(w + r[0], 0xFF, r[1] - r[0], st) != hipSuccess) rc = MEGA_MOE_ERR_HIP;
        const uint64_t comb_end = L.gemm1_out ? L.gemm1_out : L.sched;
        if (!rc && hipMemsetAsync(w + L.comb, 0xFF, comb_end - L.comb, st) != hipSuccess) rc = MEGA_MOE_ERR_HIP;
        if (rc) return rc;
    }
    mark(0);
    for (int i = 0; i < MEGA_MOE_NUM_STAGES; ++i) {
        if (on[i] && !rc) {
            hipError_t e = hipSuccess;
            switch (i) {
                case 0: e = mm::launch_route(p, st); break;
                case 1: e = mm::launch_fill(p, num_cus, st); break;
                case 2:
                    e = all_in_one   ? mm::launch_route_fill_gemms(p, num_cus, st)
                        : one_launch ? mm::launch_gemms(p, fused_fill, num_cus, st)
                                     : mm::launch_gemm1(p, fused_fill, num_cus, st);
                    break;
                case 3: e = mm::launch_gemm2(p, num_cus, st); break;
                default: e = mm::launch_combine(p, st); break;
            }
            if (e != hipSuccess) rc = MEGA_MOE_ERR_HIP;
            ran_mask |= 1u << i;
        }
        mark(i + 1);
    }
    if (!rc && timing) {
        h->ran[set] = ran_mask;
        h->pending[set] = true;
        ++h->next_set;
    }
    return rc;
}


// ---------------------------------------------------------------- workspace for callers that cannot allocate
// mega_moe_forward_noalloc runs its forward over this array instead of a caller workspace.  Every GPU the
// library runs on holds its own copy from the library's first use there until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr uint64_t kScratchBytes = MEGA_MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    uint8_t* ptr = nullptr;      // device address of this device's `scratch`
    int num_cus = 0;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Zero n words (a kernel, not hipMemsetAsync: the call may be captured into a HIP graph).
__global__ void zero_words_kernel(uint32_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}
// Copy the forward's status bits to the caller.
__global__ void export_status_kernel(const uint32_t* status, uint32_t* out) {
    if (threadIdx.x == 0) *out = status[0];
}

}  // namespace

extern "C" {

const char* mega_moe_strerror(int32_t code) {
    switch (code) {
        case MEGA_MOE_OK: return "ok";
        case MEGA_MOE_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad stage mask)";
        case MEGA_MOE_ERR_UNSUPPORTED: return "unsupported configuration";
        case MEGA_MOE_ERR_TOO_MANY_TOKENS: return "tokens_per_shard exceeds max_tokens_per_shard";
        case MEGA_MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than mega_moe_workspace_bytes()";
        case MEGA_MOE_ERR_HIP: return "HIP runtime error";
        case MEGA_MOE_ERR_SCRATCH_TOO_SMALL:
            return "configuration's workspace exceeds the static scratch of mega_moe_forward_noalloc";
        default: return "unknown error";
    }
}

int32_t mega_moe_workspace_bytes(const mega_moe_config* cfg, uint64_t* bytes_out) {
    if (!cfg || !bytes_out) return MEGA_MOE_ERR_INVALID_ARG;
    const int32_t rc = check_config(cfg);
    if (rc) return rc;
    mega_moe_layout L;
    make_layout(cfg, &L);
    *bytes_out = L.total;
    return MEGA_MOE_OK;
}

int32_t mega_moe_pack_weights(const mega_moe_config* cfg, const void* w1, const void* w2, void* w1_packed,
                              void* w2_packed, void* stream) {
    if (!cfg || !w1 || !w2 || !w1_packed || !w2_packed) return MEGA_MOE_ERR_INVALID_ARG;
    const int32_t rc = check_config(cfg);
    if (rc) return rc;
    if (!aligned16(w1) || !aligned16(w2) || !aligned16(w1_packed) || !aligned16(w2_packed))
        return MEGA_MOE_ERR_INVALID_ARG;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return MEGA_MOE_ERR_HIP;
    // BF16 rows are packed as bytes: twice the K bytes of an FP8 row, the same 128-byte K chunks
    const int kmul = cfg->weight_format == MEGA_MOE_WEIGHTS_BF16 ? 2 : 1;
    if (mm::launch_pack(w1, w2, w1_packed, w2_packed, cfg->num_local_experts + cfg->num_shared_experts,
                        cfg->hidden * kmul, cfg->intermediate * kmul, cfg->intermediate,
                        cfg->weight_format == MEGA_MOE_WEIGHTS_MXFP4, cus, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return MEGA_MOE_ERR_HIP;
    return MEGA_MOE_OK;
}

int32_t mega_moe_pack_scales(const mega_moe_config* cfg, const void* w1_sf, const void* w2_sf, void* w1_sf_packed,
                             void* w2_sf_packed, void* stream) {
    if (!cfg || !w1_sf || !w2_sf || !w1_sf_packed || !w2_sf_packed) return MEGA_MOE_ERR_INVALID_ARG;
    const int32_t rc = check_config(cfg);
    if (rc) return rc;
    if (cfg->weight_format != MEGA_MOE_WEIGHTS_MXFP4) return MEGA_MOE_ERR_INVALID_ARG;
    auto aligned4 = [](const void* q) { return ((uintptr_t)q & 3) == 0; };
    if (!aligned4(w1_sf) || !aligned4(w2_sf) || !aligned4(w1_sf_packed) || !aligned4(w2_sf_packed))
        return MEGA_MOE_ERR_INVALID_ARG;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return MEGA_MOE_ERR_HIP;
    if (mm::launch_pack_scales(w1_sf, w2_sf, w1_sf_packed, w2_sf_packed,
                               cfg->num_local_experts + cfg->num_shared_experts, cfg->hidden, cfg->intermediate, cus,
                               static_cast<hipStream_t>(stream)) != hipSuccess)
        return MEGA_MOE_ERR_HIP;
    return MEGA_MOE_OK;
}

int32_t mega_moe_init(const mega_moe_config* cfg, void* workspace, uint64_t workspace_bytes, void* stream,
                      mega_moe_handle** out) {
    if (!cfg || !out) return MEGA_MOE_ERR_INVALID_ARG;
    *out = nullptr;
    const int32_t rc = check_config(cfg);
    if (rc) return rc;
    if (!workspace || !aligned16(workspace) || ((uintptr_t)workspace & (kAlign - 1)))
        return MEGA_MOE_ERR_INVALID_ARG;
    mega_moe_layout L;
    make_layout(cfg, &L);
    if (workspace_bytes < L.total) return MEGA_MOE_ERR_WORKSPACE_TOO_SMALL;
    mega_moe_handle* h = new (std::nothrow) mega_moe_handle();
    if (!h) return MEGA_MOE_ERR_HIP;
    h->cfg = *cfg;
    h->lay = L;
    h->ws = static_cast<uint8_t*>(workspace);
    h->ws_bytes = workspace_bytes;
    if (hipGetDevice(&h->device) != hipSuccess ||
        hipDeviceGetAttribute(&h->num_cus, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess) {
        delete h;
        return MEGA_MOE_ERR_HIP;
    }
    for (int k = 0; k < kTimingSets; ++k)
        for (int i = 0; i <= MEGA_MOE_NUM_STAGES; ++i) h->ev[k][i] = nullptr;
    for (int k = 0; k < kTimingSets; ++k) {
        for (int i = 0; i <= MEGA_MOE_NUM_STAGES; ++i) {
            if (hipEventCreate(&h->ev[k][i]) != hipSuccess) {
                mega_moe_destroy(h);
                return MEGA_MOE_ERR_HIP;
            }
        }
    }
    if (hipMemsetAsync(workspace, 0, L.total, static_cast<hipStream_t>(stream)) != hipSuccess) {
        mega_moe_destroy(h);
        return MEGA_MOE_ERR_HIP;
    }
    *out = h;
    return MEGA_MOE_OK;
}

int32_t mega_moe_forward_stages(mega_moe_handle* h, uint32_t stages, const int32_t* tokens_per_shard,
                                const void* x, const float* x_sf, const int64_t* topk_idx,
                                const float* topk_weights, const void* w1, const float* w1_sf, const void* w2,
                                const float* w2_sf, void* y, int32_t* cum_recv_stats, void* stream) {
    if (!h) return MEGA_MOE_ERR_INVALID_ARG;
    const ForwardArgs a{tokens_per_shard, x, x_sf, topk_idx, topk_weights, w1, w1_sf, w2, w2_sf, y, cum_recv_stats};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MEGA_MOE_ERR_HIP;
    if (dev != h->device && hipSetDevice(h->device) != hipSuccess) return MEGA_MOE_ERR_HIP;
    const int32_t rc = run_forward(h->cfg, h->lay, h->ws, h->num_cus, stages, a, static_cast<hipStream_t>(stream), h);
    if (dev != h->device) (void)hipSetDevice(dev);
    return rc;
}

int32_t mega_moe_forward(mega_moe_handle* h, const int32_t* tokens_per_shard, const void* x, const float* x_sf,
                         const int64_t* topk_idx, const float* topk_weights, const void* w1, const float* w1_sf,
                         const void* w2, const float* w2_sf, void* y, int32_t* cum_recv_stats, void* stream) {
    return mega_moe_forward_stages(h, MEGA_MOE_STAGE_ALL, tokens_per_shard, x, x_sf, topk_idx, topk_weights, w1,
                                   w1_sf, w2, w2_sf, y, cum_recv_stats, stream);
}


int32_t mega_moe_forward_noalloc(const mega_moe_config* cfg, const int32_t* tokens_per_shard, const void* x,
                                 const float* x_sf, const int64_t* topk_idx, const float* topk_weights,
                                 const void* w1, const float* w1_sf, const void* w2, const float* w2_sf, void* y,
                                 int32_t* cum_recv_stats, uint32_t* device_status, void* stream) {
    if (!cfg) return MEGA_MOE_ERR_INVALID_ARG;
    const int32_t rc = check_config(cfg);
    if (rc) return rc;
    // the poison fills are memsets (not for captured graphs), and the fp32 GEMM1 output is a test aid
    if (cfg->flags & (MEGA_MOE_FLAG_DEBUG_POISON | MEGA_MOE_FLAG_KEEP_GEMM1_OUTPUT)) return MEGA_MOE_ERR_UNSUPPORTED;
    if (device_status && ((uintptr_t)device_status & 3u)) return MEGA_MOE_ERR_INVALID_ARG;
    mega_moe_layout L;
    make_layout(cfg, &L);
    if (L.total > kScratchBytes) return MEGA_MOE_ERR_SCRATCH_TOO_SMALL;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MEGA_MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MEGA_MOE_ERR_UNSUPPORTED;
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&slot, dev]() {
        void* ptr = nullptr;
        slot.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (slot.err == hipSuccess)
            slot.err = hipDeviceGetAttribute(&slot.num_cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (slot.err == hipSuccess) slot.ptr = static_cast<uint8_t*>(ptr);
    });
    if (slot.err != hipSuccess || !slot.ptr) return MEGA_MOE_ERR_HIP;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* w = slot.ptr;
    // what must start at zero: the status word (latched bits) and the schedule words; every
    // other region is written by an earlier stage of the same forward before it is read
    const int sched_words = (int)((L.total - L.sched) / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, st, reinterpret_cast<uint32_t*>(w + L.status), 1);
    hipLaunchKernelGGL(zero_words_kernel, dim3((sched_words + 255) / 256 < 64 ? (sched_words + 255) / 256 : 64),
                       dim3(256), 0, st, reinterpret_cast<uint32_t*>(w + L.sched), sched_words);
    if (hipGetLastError() != hipSuccess) return MEGA_MOE_ERR_HIP;
    const ForwardArgs a{tokens_per_shard, x, x_sf, topk_idx, topk_weights, w1, w1_sf, w2, w2_sf, y, cum_recv_stats};
    const int32_t frc = run_forward(*cfg, L, w, slot.num_cus, MEGA_MOE_STAGE_ALL, a, st, nullptr);
    if (frc) return frc;
    if (device_status) {
        hipLaunchKernelGGL(export_status_kernel, dim3(1), dim3(64), 0, st,
                           reinterpret_cast<const uint32_t*>(w + L.status), device_status);
        if (hipGetLastError() != hipSuccess) return MEGA_MOE_ERR_HIP;
    }
    return MEGA_MOE_OK;
}

int32_t mega_moe_query_layout(const mega_moe_handle* h, mega_moe_layout* out) {
    if (!h || !out) return MEGA_MOE_ERR_INVALID_ARG;
    *out = h->lay;
    return MEGA_MOE_OK;
}

int32_t mega_moe_status(mega_moe_handle* h, void* stream, uint32_t* device_flags) {
    if (!h || !device_flags) return MEGA_MOE_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint32_t v = 0;
    if (hipStreamSynchronize(st) != hipSuccess) return MEGA_MOE_ERR_HIP;
    if (hipMemcpy(&v, h->ws + h->lay.status, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess)
        return MEGA_MOE_ERR_HIP;
    if (v) {
        const uint32_t zero = 0;
        if (hipMemcpy(h->ws + h->lay.status, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
            return MEGA_MOE_ERR_HIP;
    }
    *device_flags = v;
    return MEGA_MOE_OK;
}

int32_t mega_moe_set_timing(mega_moe_handle* h, int32_t enable) {
    if (!h) return MEGA_MOE_ERR_INVALID_ARG;
    // drop whatever was recorded before (waiting for it, so the events can be reused)
    for (int k = 0; k < kTimingSets; ++k) {
        if (h->pending[k] && hipEventSynchronize(h->ev[k][MEGA_MOE_NUM_STAGES]) != hipSuccess)
            return MEGA_MOE_ERR_HIP;
        h->pending[k] = false;
    }
    for (int i = 0; i < MEGA_MOE_NUM_STAGES; ++i) {
        h->sum_ms[i] = 0.0;
        h->runs[i] = 0;
    }
    h->next_set = 0;
    h->timing = enable != 0;
    return MEGA_MOE_OK;
}

int32_t mega_moe_stage_times(mega_moe_handle* h, float* ms, int32_t* count) {
    if (!h || !ms) return MEGA_MOE_ERR_INVALID_ARG;
    for (int k = 0; k < kTimingSets; ++k)
        if (h->pending[k] && fold_times(h, k) != MEGA_MOE_OK) return MEGA_MOE_ERR_HIP;
    for (int i = 0; i < MEGA_MOE_NUM_STAGES; ++i)
        ms[i] = h->runs[i] ? (float)(h->sum_ms[i] / h->runs[i]) : 0.f;
    if (count) *count = h->next_set;
    return MEGA_MOE_OK;
}

void mega_moe_destroy(mega_moe_handle* h) {
    if (!h) return;
    for (int k = 0; k < kTimingSets; ++k)
        for (int i = 0; i <= MEGA_MOE_NUM_STAGES; ++i)
            if (h->ev[k][i]) (void)hipEventDestroy(h->ev[k][i]);
    delete h;
}

}  // extern "C"
