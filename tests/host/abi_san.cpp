// Host-side validation of the C ABI under the sanitizer build (AddressSanitizer +
// UndefinedBehaviorSanitizer on the host code of the library; its device code is not built):
// every entry point with arguments that must be rejected before any launch, the workspace size
// over edge shapes, the error strings, and the bounded expert cache in planning mode (no device
// memory).  Device pointers here are fake addresses that the library never dereferences on the
// host.  Exits 0 when every call returns the documented status; a sanitizer report aborts.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "rl_moe.h"

static int fails = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++fails;                                                     \
        }                                                                \
    } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

static uint64_t matrix_bytes(int H, int I, int q) { return (uint64_t)H * I / 256 * (q == RL_QTYPE_T1 ? 57 : 74); }

struct Layer {
    std::vector<rl_expert_desc> desc;
    rl_expert_blobs b;
    Layer(int E, int H, int I, int q, int64_t arena_delta = 0) : desc(E > 0 ? E : 1) {
        const uint64_t mb = (matrix_bytes(H, I, q == RL_QTYPE_T1 ? q : RL_QTYPE_Q2B) + 3) / 4 * 4;
        for (int e = 0; e < (int)desc.size(); ++e) {
            desc[e].qtype = q;
            desc[e].reserved = 0;
            desc[e].gate_off = 3 * e * mb;
            desc[e].up_off = (3 * e + 1) * mb;
            desc[e].down_off = (3 * e + 2) * mb;
        }
        b.arena = P(0x100000);
        b.desc = (const rl_expert_desc*)P(0x200000);
        b.desc_host = desc.data();
        b.E = E;
        b.H = H;
        b.I = I;
        b.arena_bytes = (uint64_t)(3 * (int64_t)desc.size() * (int64_t)mb + arena_delta);
    }
};

static const uint16_t* X = (const uint16_t*)P(0x1000);
static const int32_t* IDS = (const int32_t*)P(0x2000);
static const float* W = (const float*)P(0x3000);
static float* OUT = (float*)P(0x4000);
static void* WS = P(0x10000);
static const size_t WSB = (size_t)1 << 40;

int main() {
    // workspace sizes
    CHECK(rl_moe_workspace_bytes(2048, 10, 512, 2048, 512) > 0);
    CHECK(rl_moe_workspace_bytes(10, 17, 8, 256, 64) == 0);
    CHECK(rl_moe_workspace_bytes(10, 0, 8, 256, 64) == 0);
    CHECK(rl_moe_workspace_bytes(10, 2, 1025, 256, 64) == 0);
    CHECK(rl_moe_workspace_bytes(10, 2, 8, 200, 64) == 0);
    CHECK(rl_moe_workspace_bytes(-1, 2, 8, 256, 64) == 0);
    CHECK(rl_moe_workspace_bytes(262144, 8, 512, 2048, 512) == 0);
    CHECK(rl_moe_workspace_bytes(0x7FFFFFFF, 16, 1024, 8192, 4096) == 0);

    Layer ok(8, 2048, 512, RL_QTYPE_T1);
    typedef int (*LayerFn)(const uint16_t*, const int32_t*, const float*, const rl_expert_blobs*, float*, int32_t,
                           int32_t, void*, size_t, void*);
    LayerFn fns[] = {rl_moe_prefill, rl_moe_decode};
    for (LayerFn f : fns) {
        CHECK(f(X, IDS, W, &ok.b, OUT, 2, 17, WS, WSB, nullptr) == RL_ESHAPE);
        CHECK(f(X, IDS, W, &ok.b, OUT, 2, 0, WS, WSB, nullptr) == RL_ESHAPE);
        CHECK(f(nullptr, IDS, W, &ok.b, OUT, 2, 2, WS, WSB, nullptr) == RL_EINVAL);
        CHECK(f(X, IDS, W, &ok.b, nullptr, 2, 2, WS, WSB, nullptr) == RL_EINVAL);
        CHECK(f((const uint16_t*)P(0x1008), IDS, W, &ok.b, OUT, 2, 2, WS, WSB, nullptr) == RL_EINVAL);
        CHECK(f(X, (const int32_t*)P(0x2002), W, &ok.b, OUT, 2, 2, WS, WSB, nullptr) == RL_EINVAL);
        CHECK(f(X, IDS, W, &ok.b, OUT, 2, 2, nullptr, WSB, nullptr) == RL_EWORKSPACE);
        CHECK(f(X, IDS, W, &ok.b, OUT, 2, 2, P(0x10010), WSB, nullptr) == RL_EWORKSPACE);
        CHECK(f(X, IDS, W, &ok.b, OUT, 2, 2, WS, 1024, nullptr) == RL_EWORKSPACE);
        CHECK(f(X, IDS, W, nullptr, OUT, 2, 2, WS, WSB, nullptr) == RL_EINVAL);
        Layer bad_e(0, 2048, 512, RL_QTYPE_T1);
        CHECK(f(X, IDS, W, &bad_e.b, OUT, 2, 2, WS, WSB, nullptr) == RL_ESHAPE);
        Layer bad_h(8, 300, 512, RL_QTYPE_T1);
        CHECK(f(X, IDS, W, &bad_h.b, OUT, 2, 2, WS, WSB, nullptr) == RL_ESHAPE);
        Layer bad_q(8, 2048, 512, 7);
        CHECK(f(X, IDS, W, &bad_q.b, OUT, 2, 2, WS, WSB, nullptr) == RL_EQTYPE);
        Layer small(8, 2048, 512, RL_QTYPE_T1, -4);  // the last matrix ends past the arena
        CHECK(f(X, IDS, W, &small.b, OUT, 2, 2, WS, WSB, nullptr) == RL_EINVAL);
    }
    CHECK(rl_moe_decode(X, IDS, W, &ok.b, OUT, 3, 2, WS, WSB, nullptr) == RL_ESHAPE);  // 1 or 2 rows only
    CHECK(rl_moe_gate_up(X, IDS, W, &ok.b, nullptr, nullptr, nullptr, 2, 2, WS, WSB, nullptr) == RL_EINVAL);
    CHECK(rl_moe_prefill_block(X, IDS, W, &ok.b, 8, W, nullptr, OUT, 2, 2, WS, WSB, nullptr) == RL_EINVAL);
    CHECK(rl_moe_prefill_block(X, IDS, W, &ok.b, 0, nullptr, nullptr, OUT, 2, 2, WS, WSB, nullptr) == RL_EINVAL);
    CHECK(rl_moe_prefill_block(X, IDS, W, &ok.b, 0, W, (const float*)P(0x5004), OUT, 2, 2, WS, WSB, nullptr) ==
          RL_EINVAL);
    CHECK(rl_moe_prefill_block(X, IDS, W, &ok.b, 0, W, nullptr, OUT, 2, 16, WS, WSB, nullptr) == RL_ESHAPE);
    CHECK(rl_moe_decode_block(X, IDS, W, &ok.b, -1, W, nullptr, OUT, 1, 2, WS, WSB, nullptr) == RL_EINVAL);
    CHECK(rl_moe_prefill_from_logits(X, W, 9, &ok.b, -1, nullptr, nullptr, OUT, (int32_t*)P(0x6000), (float*)P(0x7000),
                                     2, 2, WS, WSB, nullptr) == RL_ESHAPE);  // n_route > E
    CHECK(rl_moe_prefill_from_logits(X, W, 8, &ok.b, -1, nullptr, nullptr, OUT, nullptr, (float*)P(0x7000), 2, 2, WS,
                                     WSB, nullptr) == RL_EINVAL);
    CHECK(rl_moe_route(W, 4, 8, 9, (int32_t*)P(0x6000), (float*)P(0x7000), nullptr) == RL_ESHAPE);
    CHECK(rl_moe_route(W, 4, 1025, 2, (int32_t*)P(0x6000), (float*)P(0x7000), nullptr) == RL_ESHAPE);
    CHECK(rl_moe_route(nullptr, 4, 8, 2, (int32_t*)P(0x6000), (float*)P(0x7000), nullptr) == RL_EINVAL);
    CHECK(rl_moe_route((const float*)P(0x3002), 4, 8, 2, (int32_t*)P(0x6000), (float*)P(0x7000), nullptr) ==
          RL_EINVAL);
    CHECK(rl_moe_group_pairs(IDS, 4, 2, 0, (int32_t*)P(0x6000), (int32_t*)P(0x6100), (int32_t*)P(0x6200), WS, WSB,
                             nullptr) == RL_ESHAPE);
    CHECK(rl_moe_group_pairs(nullptr, 4, 2, 8, (int32_t*)P(0x6000), (int32_t*)P(0x6100), (int32_t*)P(0x6200), WS,
                             WSB, nullptr) == RL_EINVAL);
    CHECK(rl_moe_dequant(3, RL_DEC_STRIP, P(0x1000), 256, OUT, nullptr) == RL_EINVAL);
    CHECK(rl_moe_dequant(RL_QTYPE_T1, 7, P(0x1000), 256, OUT, nullptr) == RL_EINVAL);
    CHECK(rl_moe_prefill_noalloc(X, IDS, W, &ok.b, OUT, 4096, 10, nullptr) == RL_ETOOBIG);
    CHECK(rl_moe_prefill_noalloc(X, IDS, W, &ok.b, OUT, 2, 17, nullptr) == RL_ESHAPE);
    CHECK(rl_moe_status(nullptr, nullptr) == RL_EINVAL);
    for (int s = 1; s >= -7; --s) CHECK(rl_moe_strerror(s) != nullptr && strlen(rl_moe_strerror(s)) > 0);

    // bounded expert cache, planning mode: residency and LRU eviction without device memory
    {
        const int E = 12, H = 256, I = 256;
        const uint64_t mb = matrix_bytes(H, I, RL_QTYPE_T1);
        std::vector<rl_expert_desc> hd(E);
        for (int e = 0; e < E; ++e) {
            hd[e].qtype = RL_QTYPE_T1;
            hd[e].reserved = 0;
            hd[e].gate_off = 3 * e * ((mb + 3) / 4 * 4);
            hd[e].up_off = hd[e].gate_off + (mb + 3) / 4 * 4;
            hd[e].down_off = hd[e].up_off + (mb + 3) / 4 * 4;
        }
        std::vector<uint8_t> arena(3 * E * ((mb + 3) / 4 * 4));
        CHECK(rl_cache_slot_bytes(H, I) >= 3 * mb);
        CHECK(rl_cache_slot_bytes(300, I) == 0);
        rl_cache* c = nullptr;
        CHECK(rl_cache_create(arena.data(), arena.size(), hd.data(), E, H, I, nullptr, 4, nullptr, &c) == RL_OK);
        CHECK(c != nullptr);
        const int32_t a[] = {0, 1, 2, 1}, b[] = {3, 0}, d[] = {4, 5, 6, 7, 8}, bad[] = {12};
        CHECK(rl_cache_prepare(c, a, 4, nullptr, nullptr) == RL_OK);
        CHECK(rl_cache_prepare(c, b, 2, nullptr, nullptr) == RL_OK);  // 3 into the free slot
        const int32_t e2[] = {4};
        CHECK(rl_cache_prepare(c, e2, 1, nullptr, nullptr) == RL_OK);  // evicts 1 (least recent)
        CHECK(rl_cache_slot_of(c, 1) == -1 && rl_cache_slot_of(c, 4) >= 0);
        CHECK(rl_cache_prepare(c, d, 5, nullptr, nullptr) == RL_ETOOBIG);
        CHECK(rl_cache_prepare(c, bad, 1, nullptr, nullptr) == RL_EINVAL);
        int64_t st[4] = {0, 0, 0, 0};
        CHECK(rl_cache_stats(c, st) == RL_OK);
        CHECK(st[2] == 5 && st[3] == 1);
        rl_cache_destroy(c);
        CHECK(rl_cache_create(arena.data(), arena.size(), hd.data(), E, H, I, nullptr, E + 1, nullptr, &c) != RL_OK);
    }

    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("ABI host validation under the sanitizers: all checks passed\n");
    return 0;
}
