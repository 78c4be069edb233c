// Host-side checks of the C ABI built with AddressSanitizer (host code only) and run on a machine
// without a GPU: every validation and error path that needs no device, plus an init that reaches the
// HIP runtime and must fail cleanly (no leak, no stray write) when no device is present.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/mega_moe.h"

static int failures = 0;
#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static mega_moe_config base() {
    mega_moe_config c;
    memset(&c, 0, sizeof(c));
    c.num_shards = 8;
    c.max_tokens_per_shard = 128;
    c.hidden = 7168;
    c.intermediate = 2048;
    c.num_experts = 256;
    c.num_local_experts = 32;
    c.local_rank = 0;
    c.topk = 8;
    c.block_m = 64;
    return c;
}

int main() {
    uint64_t bytes = 0, b2 = 0;
    mega_moe_config c = base();
    CHECK(mega_moe_workspace_bytes(&c, &bytes) == MEGA_MOE_OK && bytes > 0 && bytes % 256 == 0);
    CHECK(mega_moe_workspace_bytes(nullptr, &bytes) == MEGA_MOE_ERR_INVALID_ARG);
    CHECK(mega_moe_workspace_bytes(&c, nullptr) == MEGA_MOE_ERR_INVALID_ARG);
    c.num_shared_experts = 1;
    CHECK(mega_moe_workspace_bytes(&c, &b2) == MEGA_MOE_OK && b2 > bytes);
    c.block_m = 0;
    CHECK(mega_moe_workspace_bytes(&c, &b2) == MEGA_MOE_OK);

    // every field outside its range is rejected
    struct Bad { const char* what; void (*set)(mega_moe_config&); };
    const Bad bad[] = {
        {"shards 0", [](mega_moe_config& x) { x.num_shards = 0; }},
        {"shards 65", [](mega_moe_config& x) { x.num_shards = 65; }},
        {"tokens 0", [](mega_moe_config& x) { x.max_tokens_per_shard = 0; }},
        {"hidden 128", [](mega_moe_config& x) { x.hidden = 128; }},
        {"hidden 300", [](mega_moe_config& x) { x.hidden = 300; }},
        {"hidden 16640", [](mega_moe_config& x) { x.hidden = 16640; }},
        {"inter 64", [](mega_moe_config& x) { x.intermediate = 64; }},
        {"inter 200", [](mega_moe_config& x) { x.intermediate = 200; }},
        {"experts 0", [](mega_moe_config& x) { x.num_experts = 0; }},
        {"experts 250", [](mega_moe_config& x) { x.num_experts = 250; }},
        {"local 0", [](mega_moe_config& x) { x.num_local_experts = 0; }},
        {"local 2048", [](mega_moe_config& x) { x.num_local_experts = 2048; }},
        {"rank 8", [](mega_moe_config& x) { x.local_rank = 8; }},
        {"rank -1", [](mega_moe_config& x) { x.local_rank = -1; }},
        {"topk 0", [](mega_moe_config& x) { x.topk = 0; }},
        {"topk 65", [](mega_moe_config& x) { x.topk = 65; }},
        {"block_m 96", [](mega_moe_config& x) { x.block_m = 96; }},
        {"flags", [](mega_moe_config& x) { x.flags = 0x80; }},
        {"shared 2", [](mega_moe_config& x) { x.num_shared_experts = 2; }},
        {"shared, topk 64", [](mega_moe_config& x) { x.num_shared_experts = 1; x.topk = 64; }},
        {"tokens*topk overflow", [](mega_moe_config& x) { x.max_tokens_per_shard = 1 << 30; x.topk = 4; }},
    };
    for (const Bad& b : bad) {
        mega_moe_config x = base();
        b.set(x);
        const int32_t rc = mega_moe_workspace_bytes(&x, &bytes);
        if (rc != MEGA_MOE_ERR_UNSUPPORTED) {
            fprintf(stderr, "%s: got %d\n", b.what, rc);
            ++failures;
        }
    }
    for (int32_t code = -6; code <= 0; ++code) CHECK(mega_moe_strerror(code) && strlen(mega_moe_strerror(code)) > 0);

    // argument checks before any HIP call
    c = base();
    mega_moe_workspace_bytes(&c, &bytes);
    mega_moe_handle* h = (mega_moe_handle*)0x1;
    void* ws = aligned_alloc(256, 4096);
    CHECK(mega_moe_init(nullptr, ws, bytes, nullptr, &h) == MEGA_MOE_ERR_INVALID_ARG);
    CHECK(mega_moe_init(&c, ws, bytes, nullptr, nullptr) == MEGA_MOE_ERR_INVALID_ARG);
    CHECK(mega_moe_init(&c, nullptr, bytes, nullptr, &h) == MEGA_MOE_ERR_INVALID_ARG && h == nullptr);
    CHECK(mega_moe_init(&c, (char*)ws + 8, bytes, nullptr, &h) == MEGA_MOE_ERR_INVALID_ARG);
    CHECK(mega_moe_init(&c, ws, bytes - 1, nullptr, &h) == MEGA_MOE_ERR_WORKSPACE_TOO_SMALL);
    CHECK(mega_moe_pack_weights(&c, nullptr, ws, ws, ws, nullptr) == MEGA_MOE_ERR_INVALID_ARG);
    CHECK(mega_moe_pack_weights(&c, (char*)ws + 4, ws, ws, ws, nullptr) == MEGA_MOE_ERR_INVALID_ARG);
    // exponent transform: MXFP4 configs only; null and misaligned pointers rejected before any device work
    CHECK(mega_moe_pack_scales(&c, ws, ws, ws, ws, nullptr) == MEGA_MOE_ERR_INVALID_ARG);
    {
        mega_moe_config mx = c;
        mx.weight_format = MEGA_MOE_WEIGHTS_MXFP4;
        CHECK(mega_moe_pack_scales(&mx, nullptr, ws, ws, ws, nullptr) == MEGA_MOE_ERR_INVALID_ARG);
        CHECK(mega_moe_pack_scales(&mx, ws, (char*)ws + 2, ws, ws, nullptr) == MEGA_MOE_ERR_INVALID_ARG);
        CHECK(mega_moe_pack_scales(nullptr, ws, ws, ws, ws, nullptr) == MEGA_MOE_ERR_INVALID_ARG);
        mx.weight_format = 7;
        CHECK(mega_moe_pack_scales(&mx, ws, ws, ws, ws, nullptr) == MEGA_MOE_ERR_UNSUPPORTED);
    }
    const int32_t tps[8] = {1, 2, 3, 4, 5, 6, 7, 8};
    CHECK(mega_moe_forward(nullptr, tps, ws, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr, nullptr) == MEGA_MOE_ERR_INVALID_ARG);
    mega_moe_layout L;
    uint32_t flags = 0;
    float ms[MEGA_MOE_NUM_STAGES];
    CHECK(mega_moe_query_layout(nullptr, &L) == MEGA_MOE_ERR_INVALID_ARG);
    CHECK(mega_moe_status(nullptr, nullptr, &flags) == MEGA_MOE_ERR_INVALID_ARG);
    CHECK(mega_moe_set_timing(nullptr, 1) == MEGA_MOE_ERR_INVALID_ARG);
    CHECK(mega_moe_stage_times(nullptr, ms, nullptr) == MEGA_MOE_ERR_INVALID_ARG);
    mega_moe_destroy(nullptr);

    // a well-formed init reaches the HIP runtime; without a device it must fail and free its handle
    // (host memory stands in for the workspace: the call fails before the workspace is touched)
    void* big = aligned_alloc(256, (bytes + 255) / 256 * 256);
    const int32_t rc = mega_moe_init(&c, big, bytes, nullptr, &h);
    CHECK(rc == MEGA_MOE_ERR_HIP && h == nullptr);
    free(big);
    free(ws);
    if (failures) {
        fprintf(stderr, "%d host check(s) failed\n", failures);
        return 1;
    }
    printf("host checks ok\n");
    return 0;
}
