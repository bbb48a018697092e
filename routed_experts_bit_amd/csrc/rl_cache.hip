// Bounded expert cache (declarations and contracts: include/rl_moe.h, rl_cache_*).
//
// The layer's experts stay in host memory; a fixed set of device slots holds the ones the next
// call needs (Red Lite dev72, "The 2-row verify with a bounded expert cache": one prepare of the
// union of both rows' experts, so that one row cannot evict the other's experts while they are
// in flight).  Each slot holds one expert's gate, up and down matrices at fixed 256-byte aligned
// offsets.  The device descriptor table is updated by a small kernel whose arguments carry the
// changed entries: they are captured when the launch is enqueued (the same dev72 section: tables
// written into shared buffers at encode time gave an in-flight row another row's tables), and the
// expert bytes come from the host arena, which never changes, by asynchronous copies on the same
// stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <new>
#include <vector>

#include "rl_moe.h"

namespace {

constexpr int QT_Q2B_ = RL_QTYPE_Q2B, QT_T1_ = RL_QTYPE_T1;
constexpr uint64_t SLOT_ALIGN = 256;

uint64_t mat_bytes(int qtype, int32_t H, int32_t I) {
    return (uint64_t)H * (uint64_t)I / 256u * (uint64_t)(qtype == QT_T1_ ? 57 : 74);
}
uint64_t align256(uint64_t n) { return (n + SLOT_ALIGN - 1) / SLOT_ALIGN * SLOT_ALIGN; }

// descriptor entries set per launch: carried in the kernel arguments
constexpr int DESC_BATCH = 48;
struct DescUpdate {
    int32_t n;
    int32_t e[DESC_BATCH];
    rl_expert_desc d[DESC_BATCH];
};
static_assert(sizeof(DescUpdate) < 4000, "kernel arguments");

__global__ void k_set_desc(rl_expert_desc* __restrict__ desc, DescUpdate u) {
    const int i = threadIdx.x;
    if (i < u.n) desc[u.e[i]] = u.d[i];
}

}  // namespace

struct rl_cache {
    const uint8_t* host_arena;
    uint64_t host_bytes;
    std::vector<rl_expert_desc> host_desc;  // where each expert lives in host memory
    int32_t E, H, I;
    uint8_t* slots;                         // [n_slots][slot_bytes] device, or NULL (planning only)
    int32_t n_slots;
    uint64_t slot_bytes;
    rl_expert_desc* dev_desc;               // [E] device
    std::vector<rl_expert_desc> view_desc;  // host copy of the device table
    std::vector<int32_t> slot_expert;       // expert held by each slot, -1 if free
    std::vector<int64_t> slot_used;         // prepare count when the slot was last requested
    std::vector<int32_t> expert_slot;       // slot of each expert, -1 if not resident
    std::vector<int64_t> mark;              // prepare count when the expert was last requested
    int64_t tick = 0, hits = 0, misses = 0, evictions = 0;

    rl_expert_desc slot_desc(int32_t e, int32_t s) const {
        const uint64_t base = (uint64_t)s * slot_bytes;
        const uint64_t a = align256(mat_bytes(host_desc[e].qtype, H, I));
        rl_expert_desc d = {};
        d.qtype = host_desc[e].qtype;
        d.gate_off = base;
        d.up_off = base + a;
        d.down_off = base + 2 * a;
        return d;
    }
};

extern "C" {

uint64_t rl_cache_slot_bytes(int32_t H, int32_t I) {
    if (H < 256 || H > 8192 || H % 256 || I < 64 || I > 4096 || I % 64) return 0;
    return 3 * align256(mat_bytes(QT_Q2B_, H, I));  // the larger block type
}

int rl_cache_create(const void* host_arena, uint64_t host_arena_bytes, const rl_expert_desc* host_desc, int32_t E,
                    int32_t H, int32_t I, void* slots, int32_t n_slots, rl_expert_desc* dev_desc, rl_cache** out) {
    if (!out) return RL_EINVAL;
    *out = nullptr;
    const uint64_t sb = rl_cache_slot_bytes(H, I);
    if (E < 1 || E > 1024 || sb == 0 || n_slots < 1 || n_slots > E) return RL_ESHAPE;
    if (!host_arena || !host_desc) return RL_EINVAL;
    if (slots != nullptr && (!dev_desc || ((uintptr_t)slots % SLOT_ALIGN) || ((uintptr_t)dev_desc & 7))) return RL_EINVAL;
    for (int e = 0; e < E; ++e) {
        const rl_expert_desc& d = host_desc[e];
        if (d.qtype != QT_Q2B_ && d.qtype != QT_T1_) return RL_EQTYPE;
        const uint64_t mb = mat_bytes(d.qtype, H, I);
        const uint64_t offs[3] = {d.gate_off, d.up_off, d.down_off};
        for (uint64_t o : offs)
            if (o > host_arena_bytes || host_arena_bytes - o < mb) return RL_EINVAL;
    }
    rl_cache* c = new (std::nothrow) rl_cache();
    if (!c) return RL_EINVAL;
    c->host_arena = static_cast<const uint8_t*>(host_arena);
    c->host_bytes = host_arena_bytes;
    c->host_desc.assign(host_desc, host_desc + E);
    c->E = E;
    c->H = H;
    c->I = I;
    c->slots = static_cast<uint8_t*>(slots);
    c->n_slots = n_slots;
    c->slot_bytes = sb;
    c->dev_desc = dev_desc;
    c->slot_expert.assign(n_slots, -1);
    c->slot_used.assign(n_slots, -1);
    c->expert_slot.assign(E, -1);
    c->mark.assign(E, -1);
    // every expert's descriptor names a real slot from the start (slot 0 until it is loaded), so
    // the view always passes the layer's descriptor checks; only prepared experts are read
    c->view_desc.resize(E);
    for (int e = 0; e < E; ++e) c->view_desc[e] = c->slot_desc(e, 0);
    if (c->slots != nullptr) {
        DescUpdate u;
        for (int e0 = 0; e0 < E; e0 += DESC_BATCH) {
            u.n = E - e0 < DESC_BATCH ? E - e0 : DESC_BATCH;
            for (int i = 0; i < u.n; ++i) {
                u.e[i] = e0 + i;
                u.d[i] = c->view_desc[e0 + i];
            }
            hipLaunchKernelGGL(k_set_desc, dim3(1), dim3(64), 0, 0, c->dev_desc, u);
        }
        if (hipGetLastError() != hipSuccess || hipStreamSynchronize(0) != hipSuccess) {
            delete c;
            return RL_EHIP;
        }
    }
    *out = c;
    return RL_OK;
}

int rl_cache_prepare(rl_cache* c, const int32_t* ids, int32_t n, rl_expert_blobs* blobs, void* stream) {
    if (!c || (n > 0 && !ids)) return RL_EINVAL;
    if (n < 0) return RL_ESHAPE;
    for (int i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= c->E) return RL_EINVAL;
    const int64_t t = ++c->tick;
    // the distinct experts of the request, in first-appearance order
    std::vector<int32_t> req;
    req.reserve(n);
    for (int i = 0; i < n; ++i)
        if (c->mark[ids[i]] != t) {
            c->mark[ids[i]] = t;
            req.push_back(ids[i]);
        }
    if ((int)req.size() > c->n_slots) {
        for (int32_t e : req) c->mark[e] = -1;  // the request is refused: leave no trace of it
        --c->tick;
        return RL_ETOOBIG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    DescUpdate u;
    u.n = 0;
    auto flush = [&]() {
        if (u.n > 0 && c->slots != nullptr) hipLaunchKernelGGL(k_set_desc, dim3(1), dim3(64), 0, s, c->dev_desc, u);
        u.n = 0;
    };
    for (int32_t e : req) {
        const int32_t sl = c->expert_slot[e];
        if (sl >= 0) {
            c->slot_used[sl] = t;
            ++c->hits;
        }
    }
    for (int32_t e : req) {
        if (c->expert_slot[e] >= 0) continue;
        ++c->misses;
        // a free slot (lowest index), else the least recently requested slot outside this request
        int32_t v = -1;
        for (int32_t sl = 0; sl < c->n_slots && v < 0; ++sl)
            if (c->slot_expert[sl] < 0) v = sl;
        if (v < 0) {
            for (int32_t sl = 0; sl < c->n_slots; ++sl)
                if (c->slot_used[sl] != t && (v < 0 || c->slot_used[sl] < c->slot_used[v])) v = sl;
            c->expert_slot[c->slot_expert[v]] = -1;
            ++c->evictions;
        }
        c->slot_expert[v] = e;
        c->slot_used[v] = t;
        c->expert_slot[e] = v;
        const rl_expert_desc d = c->slot_desc(e, v);
        if (c->slots != nullptr) {
            const rl_expert_desc& h = c->host_desc[e];
            const uint64_t mb = mat_bytes(h.qtype, c->H, c->I);
            const uint64_t src[3] = {h.gate_off, h.up_off, h.down_off};
            const uint64_t dst[3] = {d.gate_off, d.up_off, d.down_off};
            for (int m = 0; m < 3; ++m)
                if (hipMemcpyAsync(c->slots + dst[m], c->host_arena + src[m], mb, hipMemcpyHostToDevice, s) != hipSuccess)
                    return RL_EHIP;
        }
        c->view_desc[e] = d;
        u.e[u.n] = e;
        u.d[u.n] = d;
        if (++u.n == DESC_BATCH) flush();
    }
    flush();
    if (blobs) {
        blobs->arena = c->slots;
        blobs->desc = c->dev_desc;
        blobs->desc_host = c->view_desc.data();
        blobs->E = c->E;
        blobs->H = c->H;
        blobs->I = c->I;
        blobs->arena_bytes = (uint64_t)c->n_slots * c->slot_bytes;
    }
    if (c->slots == nullptr) return RL_OK;  // planning only: no HIP call at all
    return hipGetLastError() == hipSuccess ? RL_OK : RL_EHIP;
}

int rl_cache_stats(const rl_cache* c, int64_t* stats) {
    if (!c || !stats) return RL_EINVAL;
    stats[0] = c->tick;
    stats[1] = c->hits;
    stats[2] = c->misses;
    stats[3] = c->evictions;
    return RL_OK;
}

int32_t rl_cache_slot_of(const rl_cache* c, int32_t e) {
    if (!c || e < 0 || e >= c->E) return -1;
    return c->expert_slot[e];
}

void rl_cache_destroy(rl_cache* c) { delete c; }

}  // extern "C"
