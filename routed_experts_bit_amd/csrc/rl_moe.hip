// C ABI of the routed-expert MoE layer (declarations and contracts: include/rl_moe.h).
//
// Host side: argument validation (synchronous, before any launch), workspace carving and
// stream-ordered launches.  No device allocation, no host synchronisation inside a call, no
// library-global device buffers: every per-call table lives in the caller's workspace (Red
// Lite dev72, "2-row verify": tables written into shared buffers at encode time let one
// in-flight row read another row's tables).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "rl_kernels.h"
#include "rl_route.h"
#include "rl_moe.h"

// Workspace of rl_moe_prefill_noalloc: one copy per device, held for the life of the process.
// Host code never uses this name as an address: each device's address comes from
// hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[RL_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace rl;

// Device address of `scratch` on the current device, looked up once per device (with that device
// current) and kept; nullptr if the runtime reports an error.
constexpr int NOALLOC_MAXDEV = 64;
std::atomic<void*> g_scratch[NOALLOC_MAXDEV];
std::mutex g_scratch_mu;

void* noalloc_scratch(bool lookup) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAXDEV) return nullptr;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p != nullptr || !lookup) return p;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t n) { return (n + ALIGN - 1) / ALIGN * ALIGN; }

struct Layout {
    size_t flags, gvpairs, offsets, pair_src, inv, tile_hist, items, xq, xscale, h8, hscale, hbuf, yslot, yexp, yspare,
        total;
    int maxrec;  // work records per block type
};

// Grouping tiles of tp pairs (tp = GT, or the largest multiple of the pairs per token that fits
// GT when the router runs in the grouping's first launch: always more than GT / 2).
int group_tiles(int64_t P, int tp = GT) { return (int)((P + tp - 1) / tp); }
int tile_hist_rows(int64_t P) { return P > 0 ? group_tiles(P, GT / 2) : 1; }

// Largest byte extent of a buffer that the kernels address with 32-bit offsets (activation rows
// of the gate/up and down GEMMs); their buffer resources span at most 0x7FFFFFF0 bytes.
constexpr int64_t OFF32_LIMIT = (int64_t(1) << 31) - (int64_t(1) << 16);

bool shape_ok(int64_t T, int32_t k, int32_t E, int32_t H, int32_t I) {
    if (T < 0 || k < 1 || k > 16) return false;
    if (E < 1 || E > MAX_E) return false;
    if (H < 256 || H > 8192 || H % 256) return false;
    if (I < 64 || I > 4096 || I % 64) return false;
    if (!(I % 256 == 0 || I == 64 || I == 128)) return false;
    const int64_t P = T * (int64_t)k;
    if (P > (1 << 24)) return false;
    // x rows (bf16, or split into hi/lo fp8: 2H bytes per token) and h rows (fp16, or split:
    // 2I bytes per pair) are read through 32-bit buffer offsets
    if (T * 2 * (int64_t)H > OFF32_LIMIT) return false;
    if (P * 2 * (int64_t)I > OFF32_LIMIT) return false;
    return true;
}

inline uint64_t matrix_bytes(int qtype, int32_t H, int32_t I) {
    return (uint64_t)H * (uint64_t)I / 256u * (uint64_t)(qtype == QT_T1 ? Fmt<QT_T1>::BYTES : Fmt<QT_Q2B>::BYTES);
}

Layout layout(int64_t T, int32_t k, int32_t E, int32_t H, int32_t I) {
    Layout L;
    const size_t P = (size_t)T * (size_t)k;
    size_t off = 0;
    L.flags = off;
    off = align_up(off + FLAGS_WORDS * sizeof(int32_t));
    L.gvpairs = off;  // the resolved pair table of the 1-2 row path
    off = align_up(off + GV_MAX_PAIRS * sizeof(GvPair));
    L.offsets = off;
    off = align_up(off + (size_t)(E + 1) * sizeof(int32_t));
    L.pair_src = off;
    off = align_up(off + P * sizeof(int32_t));
    L.inv = off;
    off = align_up(off + P * sizeof(int32_t));
    L.tile_hist = off;
    off = align_up(off + (size_t)tile_hist_rows((int64_t)P) * E * sizeof(int32_t));
    L.items = off;  // work records, [2][maxrec]
    L.maxrec = max_records(E, (int)P);
    off = align_up(off + 2 * (size_t)L.maxrec * sizeof(ItemRec));
    L.xq = off;  // fp8 hi/lo activations of the T1 path
    off = align_up(off + (size_t)T * 2 * H);
    L.xscale = off;  // scale of each row of xq
    off = align_up(off + (size_t)T * sizeof(float));
    L.h8 = off;  // fp8 hi/lo h of the T1 down path
    off = align_up(off + P * (size_t)2 * I);
    L.hscale = off;  // scale of each row of h8 (I > 512), or its four k-group scales (I <= 512)
    off = align_up(off + P * sizeof(float));
    L.hbuf = off;  // fp16 h of the prefill path, or fp32 h of the 1-2 row path
    off = align_up(off + P * (size_t)I * sizeof(float));
    L.yslot = off;  // fp16 y * 2^sigma, row t*k + j of each pair
    off = align_up(off + P * (size_t)H * sizeof(uint16_t));
    L.yexp = off;  // sigma of each (pair, 64-column tile)
    off = align_up(off + P * (size_t)(H / CT));
    L.yspare = off;  // each down wave's target for its padding rows
    off = align_up(off + (size_t)Y_SPARE * CT * sizeof(uint16_t) + Y_SPARE);
    L.total = off;
    return L;
}

int hip_status() { return hipGetLastError() == hipSuccess ? RL_OK : RL_EHIP; }

template <typename P>
P* at(void* ws, size_t off) {
    return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

// Common validation of the layer entry points.  Fills `present[q]` with the number of
// experts of type q (from the host copy of the descriptors).  The workspace is checked last
// (check_ws), so that callers can check buffers of their own in between.
int check_ws(const rl_expert_blobs* ex, int32_t T, int32_t k, const void* ws, size_t ws_bytes) {
    if (!ws || ((uintptr_t)ws % ALIGN)) return RL_EWORKSPACE;
    if (ws_bytes < layout(T, k, ex->E, ex->H, ex->I).total) return RL_EWORKSPACE;
    return RL_OK;
}

// The pairs of a call: kin selections per token from topk_ids / topk_w, plus (shared >= 0) one
// pair of the shared expert per token weighted by gate[t]; res (may be NULL) is added to out
// after the ordered sum.
// With logits != NULL the call routes first: the router picks the kin selections of every token
// among experts [0, n_route) from logits [T][n_route] and writes them to ids / w (the caller's
// output buffers), in the grouping's first launch.
struct Route {
    const int32_t* ids;
    const float* w;
    int32_t kin;
    int32_t shared;
    const float* gate;
    const float* res;
    const float* logits = nullptr;
    int32_t n_route = 0;
    int32_t kk() const { return kin + (shared >= 0 ? 1 : 0); }
    PairIds pid() const { return PairIds{ids, kin, kk(), shared}; }
};
inline Route routed_only(const int32_t* ids, const float* w, int32_t k) { return Route{ids, w, k, -1, nullptr, nullptr}; }

int check_args(const void* x, const Route& r, const rl_expert_blobs* ex, const void* out, int32_t T, int present[3]) {
    if (!ex) return RL_EINVAL;
    if (r.kin < 0 || !shape_ok(T, r.kk(), ex->E, ex->H, ex->I)) return RL_ESHAPE;
    if (r.shared >= ex->E) return RL_EINVAL;
    if (r.logits != nullptr && (r.n_route < 1 || r.n_route > ex->E || r.kin < 1 || r.kin > r.n_route)) return RL_ESHAPE;
    if (T == 0) return RL_OK;
    if ((uintptr_t)r.logits & 3) return RL_EINVAL;
    if (!x || !out || !ex->arena || !ex->desc || !ex->desc_host) return RL_EINVAL;
    if (r.kin > 0 && (!r.ids || !r.w)) return RL_EINVAL;
    if (r.shared >= 0 && !r.gate) return RL_EINVAL;
    // the kernels move x, out and the residual in 16-byte pieces and ids, w, gates and
    // descriptors in 4- and 8-byte words
    if (((uintptr_t)x | (uintptr_t)out | (uintptr_t)r.res) & 15) return RL_EINVAL;
    if (((uintptr_t)r.ids | (uintptr_t)r.w | (uintptr_t)r.gate) & 3) return RL_EINVAL;
    if ((uintptr_t)ex->desc & 7) return RL_EINVAL;
    if ((uintptr_t)ex->arena & 3) return RL_EINVAL;
    present[0] = present[1] = present[2] = 0;
    for (int e = 0; e < ex->E; ++e) {
        const rl_expert_desc& dd = ex->desc_host[e];
        int q = dd.qtype;
        if (q != QT_Q2B && q != QT_T1) return RL_EQTYPE;
        if ((dd.gate_off | dd.up_off | dd.down_off) & 3) return RL_EINVAL;
        // every matrix inside the arena (the kernels' reads stay inside its matrix's dwords)
        const uint64_t mb = matrix_bytes(q, ex->H, ex->I);
        const uint64_t offs[3] = {dd.gate_off, dd.up_off, dd.down_off};
        for (uint64_t o : offs)
            if (o > ex->arena_bytes || ex->arena_bytes - o < mb) return RL_EINVAL;
        present[q] += 1;
    }
    return RL_OK;
}

int check_layer(const void* x, const Route& r, const rl_expert_blobs* ex, const void* out, int32_t T, const void* ws,
                size_t ws_bytes, int present[3]) {
    const int rc = check_args(x, r, ex, out, T, present);
    if (rc != RL_OK || T == 0) return rc;
    return check_ws(ex, T, r.kk(), ws, ws_bytes);
}

// Pair grouping; with split != NULL the split of x runs in the histogram launch.
void launch_group(const PairIds& pid, int32_t T, int32_t E, const rl_expert_desc* desc, int32_t* offsets,
                  int32_t* pair_src, int32_t* inv, int32_t* flags, int32_t* tile_hist, ItemRec* items, int maxrec,
                  hipStream_t s, const SplitArgs* split = nullptr, void* zero = nullptr, size_t zero_bytes = 0) {
    GroupArgs g;
    g.zero = static_cast<u32x4*>(zero);
    g.nzero = zero != nullptr ? (int)(zero_bytes / 16) : 0;
    g.pid = pid;
    g.desc = desc;
    g.offsets = offsets;
    g.pair_src = pair_src;
    g.inv = inv;
    g.flags = flags;
    g.items = items;
    g.maxrec = maxrec;
    g.tile_hist = tile_hist;
    g.P = T * pid.kk;
    g.E = E;
    g.tp = GT;
    g.ntiles = group_tiles(g.P) > 0 ? group_tiles(g.P) : 1;
    g.nflags = FLAGS_WORDS;
    const int nsplit = split != nullptr && split->rows > 0 ? split->rows : 0;
    const int G = split != nullptr ? split->K / 32 : 8;  // K <= 8192: G <= 256
    if (nsplit > 0) {
        const SplitArgs& a = *split;
#define RL_CSPLIT(LPR, NG)                                                                                      \
    hipLaunchKernelGGL((k_count_split<LPR, NG>), dim3(g.ntiles + (a.rows + 256 / LPR - 1) / (256 / LPR)), \
                       dim3(256), 0, s, g, a)
        if (G <= 8)
            RL_CSPLIT(8, 1);
        else if (G <= 16)
            RL_CSPLIT(16, 1);
        else if (G <= 32)
            RL_CSPLIT(32, 1);
        else if (G <= 64)
            RL_CSPLIT(64, 1);
        else if (G <= 128)
            RL_CSPLIT(64, 2);
        else if (G <= 192)
            RL_CSPLIT(64, 3);
        else
            RL_CSPLIT(64, 4);
#undef RL_CSPLIT
    } else {
        hipLaunchKernelGGL(k_group_count, dim3(g.ntiles), dim3(GROUP_NTHR), 0, s, g);
    }
    hipLaunchKernelGGL(k_group_scatter, dim3(g.ntiles + 1), dim3(GROUP_NTHR), 0, s, g);  // + the lister
}

// Persistent grids: as many work-groups as fit on the device at once (occupancy query, cached
// per kernel), a multiple of 8 so that every XCD gets the same number.
template <auto K>
int resident_grid(int block) {
    // per device (the current one), computed once; concurrent first calls compute the same value
    constexpr int MAXDEV = 64;
    static std::atomic<int> cached[MAXDEV];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    std::atomic<int>& slot = cached[dev < MAXDEV ? dev : MAXDEV - 1];
    int grid = slot.load(std::memory_order_relaxed);
    if (grid == 0) {
        int cus = 256, per_cu = 1;
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, K, block, 0) != hipSuccess || per_cu < 1) per_cu = 1;
        grid = ((cus * per_cu + 7) / 8) * 8;
        slot.store(grid, std::memory_order_relaxed);
    }
    return grid;
}

int grid_cap(int grid, int n_experts, int ns) {
    const int items = ((n_experts + 7) / 8) * 8 * ns;
    return grid < items ? grid : items;
}

// Down launches (4 waves per work-group) give every wave its own spare y tile: at most
// Y_SPARE / 4 work-groups (a multiple of 8; MI355X holds 512 of them at once).
int down_grid(int grid) { return grid < Y_SPARE / 4 ? grid : Y_SPARE / 4; }

// The LDS-window kernels of a block type (T1 on the fp8 MFMA, Q2B on the 16-bit MFMA).
template <int QT, int MODE, int NTI, bool SPAN = false>
constexpr auto mm_kernel() {
    if constexpr (QT == QT_T1)
        return &k_t1_f8<MODE, NTI, SPAN>;
    else
        return &k_q2_mm<MODE, NTI, SPAN>;
}
template <int QT>
constexpr auto dn_kernel_of() {
    if constexpr (QT == QT_T1)
        return &k_t1_dn;
    else
        return &k_q2_dn;
}

template <int QT, int MODE, int NTI, bool SPAN = false>
void launch_mm(const GuArgs& b, int n_experts, hipStream_t s) {
    constexpr auto K = mm_kernel<QT, MODE, NTI, SPAN>();
    const int grid = grid_cap(resident_grid<K>(64 * GU_NW), n_experts, b.ns);
    hipLaunchKernelGGL(K, dim3(grid), dim3(64 * GU_NW), 0, s, b);
}

// Whether every expert of block type qt has its gate and up matrices within one buffer resource
// (the span from the lower to the end of the higher below 2^31 bytes), so that the T1 gate/up
// kernel can fetch the windows of both with one instruction.
bool gateup_spans(const rl_expert_blobs* ex, int qt) {
    const uint64_t mb = matrix_bytes(qt, ex->H, ex->I);
    for (int e = 0; e < ex->E; ++e) {
        const rl_expert_desc& d = ex->desc_host[e];
        if (d.qtype != qt) continue;
        const uint64_t lo = d.gate_off < d.up_off ? d.gate_off : d.up_off;
        const uint64_t hi = d.gate_off < d.up_off ? d.up_off : d.gate_off;
        if (hi - lo + mb > 0x7FFF0000ull) return false;
    }
    return true;
}

// Gate/up: 4 waves x (2 gate + 2 up tiles) = 128 intermediate columns per work item when
// I % 128 == 0, else 64 columns (1 + 1 tiles per wave).
template <int QT>
void launch_gateup_mm(const GuArgs& a, int n_experts, hipStream_t s, bool span) {
    GuArgs b = a;
    if (a.N % 128 == 0) {
        b.ns = a.N / 128;
        if (span)
            launch_mm<QT, GU_GATEUP, 2, true>(b, n_experts, s);
        else
            launch_mm<QT, GU_GATEUP, 2>(b, n_experts, s);
    } else {
        b.ns = a.N / 64;
        launch_mm<QT, GU_GATEUP, 1>(b, n_experts, s);
    }
}

// Split of activation rows into hi/lo fp8 (k_split): LPR lanes per row, NG groups of 32 values
// per lane; K <= 8192.
template <int MODE>
void launch_split(const SplitArgs& a, hipStream_t s) {
    if (a.rows <= 0) return;
    const int G = a.K / 32;
#define RL_SPLIT(LPR, NG) \
    hipLaunchKernelGGL((k_split<MODE, LPR, NG>), dim3((a.rows + 256 / LPR - 1) / (256 / LPR)), dim3(256), 0, s, a)
    if (G <= 8)
        RL_SPLIT(8, 1);
    else if (G <= 16)
        RL_SPLIT(16, 1);
    else if (G <= 32)
        RL_SPLIT(32, 1);
    else if (G <= 64)
        RL_SPLIT(64, 1);
    else if (G <= 128)
        RL_SPLIT(64, 2);
    else if (G <= 192)
        RL_SPLIT(64, 3);
    else
        RL_SPLIT(64, 4);
#undef RL_SPLIT
}

// Split of h into hi/lo fp8 rows for the T1 down kernels.
void launch_hsplit(const GuArgs& a, int P, hipStream_t s) {
    SplitArgs sa = {};
    sa.src = a.hbuf;
    sa.dst = const_cast<uint8_t*>(a.act);
    sa.rows = P;
    sa.K = a.K;
    sa.scale = const_cast<float*>(a.ascale);
    launch_split<SPLIT_H>(sa, s);
}
// Columns of H per work item of the LDS-held down kernel (I a multiple of 256, at most 512).
// (512 columns: four items per work-group at 2048 columns and 512 experts, so records of
// different sizes even out; with items of 1024 columns the down kernel of the mixed-type layer
// took 117 against 102 us, of the Zipf-routed Q2B layer 86 against 81 us)
int down_item_cols(int32_t H) { return H % 512 == 0 ? 512 : 256; }

// Down on the LDS-window kernels (I a multiple of 256): for I <= 512 the activations are held in
// LDS, items of up to 1024 columns; else 4 waves x 4 tiles = 256 output columns per item.
template <int QT>
void launch_down_mm(const GuArgs& a, int n_experts, hipStream_t s) {
    GuArgs b = a;
    if (a.K <= DN_KMAX) {
        const int cw = down_item_cols(a.N);
        b.ns = a.N / cw;
        constexpr auto K = dn_kernel_of<QT>();
        const int grid = down_grid(grid_cap(resident_grid<K>(64 * GU_NW), n_experts, b.ns));
        hipLaunchKernelGGL(K, dim3(grid), dim3(64 * GU_NW), 0, s, b);
        return;
    }
    b.ns = a.N / 256;
    constexpr auto K = mm_kernel<QT, GU_DOWN, 4>();
    const int grid = down_grid(grid_cap(resident_grid<K>(64 * GU_NW), n_experts, b.ns));
    hipLaunchKernelGGL(K, dim3(grid), dim3(64 * GU_NW), 0, s, b);
}

template <int QT>
void launch_down_t(const DownArgs& a, int n_experts, hipStream_t s) {
    // 4 waves x 4 strips of 16 columns: one 64-column combine tile per wave, 256 columns per item
    DownArgs b = a;
    b.ns = a.H / 256;
    if (a.I % 256 == 0) {
        const int grid = down_grid(grid_cap(resident_grid<k_down<QT, 256, 4, 4>>(256), n_experts, b.ns));
        hipLaunchKernelGGL((k_down<QT, 256, 4, 4>), dim3(grid), dim3(256), 0, s, b);
    } else if (a.I == 128) {
        const int grid = down_grid(grid_cap(resident_grid<k_down<QT, 128, 4, 4>>(256), n_experts, b.ns));
        hipLaunchKernelGGL((k_down<QT, 128, 4, 4>), dim3(grid), dim3(256), 0, s, b);
    } else {
        const int grid = down_grid(grid_cap(resident_grid<k_down<QT, 64, 4, 4>>(256), n_experts, b.ns));
        hipLaunchKernelGGL((k_down<QT, 64, 4, 4>), dim3(grid), dim3(256), 0, s, b);
    }
}

// ordered combine, one kernel instance per number of pairs per token (1..16)
template <int K>
void launch_combine_k(const YSlots& ys, const CombineW& cw, float* out, int T, hipStream_t s) {
    hipLaunchKernelGGL(k_combine<K>, dim3(T), dim3(256), 0, s, ys, cw, out);
}
void launch_combine(const YSlots& ys, const CombineW& cw, float* out, int T, int kk, hipStream_t s) {
    switch (kk) {
#define RL_CB(K) \
    case K: launch_combine_k<K>(ys, cw, out, T, s); break;
        RL_CB(1) RL_CB(2) RL_CB(3) RL_CB(4) RL_CB(5) RL_CB(6) RL_CB(7) RL_CB(8)
        RL_CB(9) RL_CB(10) RL_CB(11) RL_CB(12) RL_CB(13) RL_CB(14) RL_CB(15) RL_CB(16)
#undef RL_CB
        default: break;  // checked to be in [1, 16] before any launch
    }
}

// 1-2 row kernels: each of the 16 lanes of a row takes d/16 consecutive values in strips of the
// widest of 64, 32 and 16 values that divides them (a strip stays inside one block and one
// sub-scale group); gate/up holds up to 8 strips per lane (H), down up to 4 per round (I).
constexpr int gv_strip(int d) { return (d / 16) % 64 == 0 ? 64 : ((d / 16) % 32 == 0 ? 32 : 16); }
constexpr int gv_nst(int d) { return d / 16 / gv_strip(d); }
bool gv_dim_ok(int d, int max_nst) { return d >= 256 && d % 256 == 0 && gv_nst(d) <= max_nst; }
constexpr int gv_maxs(int nst) { return nst <= 1 ? 1 : (nst <= 2 ? 2 : (nst <= 4 ? 4 : 8)); }

template <int QMASK>
void launch_gv(const GvArgs& a, hipStream_t s) {
    // Work-groups of 256 threads.  Every work-group copies its decode tables into LDS; with the
    // full value tables (T1 17 KB, Q2B 32 KB, both 49 KB) work-groups of 512 threads had been
    // faster for Q2B and mixed layers, with the unit rows (3-5 KB) 256 threads are as fast or
    // faster for every type mask.
    constexpr int NT = 256, NW = NT / 64;
    const int waves1 = a.R * a.k * (a.I / 2);
    const int waves2 = a.R * a.H;
    dim3 g1((waves1 + NW - 1) / NW < 1024 ? (waves1 + NW - 1) / NW : 1024);
    auto g2 = [&](int nw) { return dim3((waves2 + nw - 1) / nw < 1024 ? (waves2 + nw - 1) / nw : 1024); };
    const size_t xs_bytes = gv_xs_bytes(a.R, a.H);  // x staged in LDS (at most 32.5 KB)
#define RL_GV1(S, M) hipLaunchKernelGGL((k_gv_gateup<QMASK, S, M, NT>), g1, dim3(NT), xs_bytes, s, a)
#define RL_GV1S(S)                      \
    switch (gv_maxs(gv_nst(a.H))) {     \
        case 1: RL_GV1(S, 1); break;    \
        case 2: RL_GV1(S, 2); break;    \
        case 4: RL_GV1(S, 4); break;    \
        default: RL_GV1(S, 8); break;   \
    }
    if (gv_strip(a.H) == 64) {
        RL_GV1S(64)
    } else if (gv_strip(a.H) == 32) {
        RL_GV1S(32)
    } else {
        RL_GV1S(16)
    }
#undef RL_GV1S
#undef RL_GV1
#define RL_GV2(S, M) hipLaunchKernelGGL((k_gv_down<QMASK, S, M, NT>), g2(NW), dim3(NT), 0, s, a)
#define RL_GV2S(S)                      \
    switch (gv_maxs(gv_nst(a.I))) {     \
        case 1: RL_GV2(S, 1); break;    \
        case 2: RL_GV2(S, 2); break;    \
        default: RL_GV2(S, 4); break;   \
    }
    if (gv_strip(a.I) == 64) {
        RL_GV2S(64)
    } else if (gv_strip(a.I) == 32) {
        RL_GV2S(32)
    } else {
        RL_GV2S(16)
    }
#undef RL_GV2S
#undef RL_GV2
}

// The T1 gate/up kernel writes h already split into hi/lo fp8 rows for the fp8 down kernel that
// holds a chunk's activations in LDS (I a multiple of 256, at most DN_KMAX).
bool t1_splits_h(const int present[3], int32_t I) { return present[QT_T1] > 0 && I % 256 == 0 && I <= DN_KMAX; }

// The router: one wave per token, NR logits per lane.
void launch_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids, float* w, hipStream_t s) {
    const dim3 grid((unsigned)((T + 3) / 4));
#define RL_RT(NR) hipLaunchKernelGGL(k_route<NR>, grid, dim3(256), 0, s, logits, T, E, k, ids, w)
    if (E <= 64)
        RL_RT(1);
    else if (E <= 128)
        RL_RT(2);
    else if (E <= 256)
        RL_RT(4);
    else if (E <= 512)
        RL_RT(8);
    else
        RL_RT(16);
#undef RL_RT
}

// Upper bound of the work records of one block type (its experts, plus one per REC_HOT pairs).
int records_bound(int n_experts, int64_t P) { return n_experts + (int)((P + REC_HOT - 1) / REC_HOT); }

// grouping + gate/up for every present type; returns the layout used.  With h8 (T1, I <= 512)
// the T1 gate/up writes its h rows split for the fp8 down kernel (h8, with k-group scales hsc)
// instead of fp16 rows of hdst.
void run_group_gateup(const uint16_t* x, const Route& r, const rl_expert_blobs* ex, int32_t T, void* ws,
                      const int present[3], uint16_t* hdst, hipStream_t s, Layout& L, void* const* events = nullptr,
                      uint8_t* h8 = nullptr, uint32_t* hsc = nullptr) {
    auto mark = [&](int i) {
        if (events) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
    };
    const int kk = r.kk();
    L = layout(T, kk, ex->E, ex->H, ex->I);
    int32_t* flags = at<int32_t>(ws, L.flags);
    int32_t* pair_src = at<int32_t>(ws, L.pair_src);
    ItemRec* items = at<ItemRec>(ws, L.items);
    uint8_t* xq = at<uint8_t>(ws, L.xq);
    float* xscale = at<float>(ws, L.xscale);
    SplitArgs sa = {};  // the T1 path's split of x, in the grouping's first launch
    sa.src = x;
    sa.dst = xq;
    sa.scale = xscale;
    sa.rows = T;
    sa.K = ex->H;
    if (r.logits != nullptr)  // the router writes the call's selections first
        launch_route(r.logits, T, r.n_route, r.kin, const_cast<int32_t*>(r.ids), const_cast<float*>(r.w), s);
    launch_group(r.pid(), T, ex->E, ex->desc, at<int32_t>(ws, L.offsets), pair_src, at<int32_t>(ws, L.inv), flags,
                 at<int32_t>(ws, L.tile_hist), items, L.maxrec, s, present[QT_T1] ? &sa : nullptr,
                 at<void>(ws, L.yexp), L.yspare - L.yexp);
    mark(1);
    const int64_t P = (int64_t)T * kk;
    GuArgs b = {};
    b.pair_src = pair_src;
    b.k = kk;
    b.P = (int)P;
    b.arena = static_cast<const uint8_t*>(ex->arena);
    b.hbuf = hdst;
    b.K = ex->H;
    b.N = ex->I;
    b.ns = 1;
    if (present[QT_Q2B]) {  // x as it is (bf16)
        GuArgs q = b;
        q.act = reinterpret_cast<const uint8_t*>(x);
        q.items = items + (size_t)(QT_Q2B - 1) * L.maxrec;
        q.wl_len = flags + 8 + QT_Q2B;
        launch_gateup_mm<QT_Q2B>(q, records_bound(present[QT_Q2B], P), s, gateup_spans(ex, QT_Q2B));
    }
    if (present[QT_T1]) {  // the split of x
        GuArgs q = b;
        q.act = xq;
        q.ascale = xscale;
        q.h8 = h8;
        q.hsc = hsc;
        q.items = items + (size_t)(QT_T1 - 1) * L.maxrec;
        q.wl_len = flags + 8 + QT_T1;
        launch_gateup_mm<QT_T1>(q, records_bound(present[QT_T1], P), s, gateup_spans(ex, QT_T1));
    }
    mark(2);
}

int prefill_impl(const uint16_t* x, const Route& r, const rl_expert_blobs* experts, float* out, int32_t T,
                 void* workspace, size_t ws_bytes, void* stream, void* const* events) {
    int present[3] = {0, 0, 0};
    int rc = check_layer(x, r, experts, out, T, workspace, ws_bytes, present);
    if (rc != RL_OK || T == 0) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto mark = [&](int i) {
        if (events) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
    };
    const int kk = r.kk();
    const int64_t P = (int64_t)T * kk;
    const Layout L = layout(T, kk, experts->E, experts->H, experts->I);
    uint16_t* hbuf = at<uint16_t>(workspace, L.hbuf);
    int32_t* flags = at<int32_t>(workspace, L.flags);
    int32_t* pair_src = at<int32_t>(workspace, L.pair_src);
    ItemRec* items = at<ItemRec>(workspace, L.items);
    YSlots ys;
    ys.yslot = at<uint16_t>(workspace, L.yslot);
    ys.yexp = at<int8_t>(workspace, L.yexp);
    ys.yspare = at<uint16_t>(workspace, L.yspare);
    ys.espare = at<int8_t>(workspace, L.yspare + (size_t)Y_SPARE * CT * sizeof(uint16_t));
    ys.H = experts->H;
    ys.P = (int)P;
    mark(0);
    Layout L2;  // same layout as L
    // T1 with I <= 512: gate/up writes h already split for the down kernel (no split of h)
    const bool t1_hsplit_fused = t1_splits_h(present, experts->I);
    uint8_t* h8 = at<uint8_t>(workspace, L.h8);
    uint32_t* hsc = at<uint32_t>(workspace, L.hscale);
    run_group_gateup(x, r, experts, T, workspace, present, hbuf, s, L2, events, t1_hsplit_fused ? h8 : nullptr,
                     t1_hsplit_fused ? hsc : nullptr);
    DownArgs d;
    d.hbuf = hbuf;
    d.arena = static_cast<const uint8_t*>(experts->arena);
    d.pair_src = pair_src;
    d.ys = ys;
    d.flags = flags;
    d.H = experts->H;
    d.I = experts->I;
    d.ns = 1;
    // I a multiple of 256: the LDS-window down kernels (T1 reads h split into hi/lo fp8, Q2B reads
    // h as it is); I = 64 or 128: k_down
    const bool mm_dn = experts->I % 256 == 0;
    GuArgs b = {};
    b.pair_src = pair_src;
    b.arena = d.arena;
    b.hbuf = hbuf;
    b.ys = ys;
    b.flags = flags;
    b.K = experts->I;
    b.N = experts->H;
    b.P = (int)P;
    if (mm_dn && present[QT_T1]) {
        b.act = h8;
        b.ascale = at<float>(workspace, L.hscale);  // I > 512: one scale per row, from the split of h
        b.hsc = hsc;                                // I <= 512: k-group scales from gate/up
        if (!t1_hsplit_fused) launch_hsplit(b, (int)P, s);
    }
    mark(3);
    for (int q = QT_Q2B; q <= QT_T1; ++q) {
        if (!present[q]) continue;
        const int nrec = records_bound(present[q], P);
        if (mm_dn) {
            GuArgs bq = b;
            bq.items = items + (size_t)(q - 1) * L.maxrec;
            bq.wl_len = flags + 8 + q;
            if (q == QT_Q2B) {
                bq.act = reinterpret_cast<const uint8_t*>(hbuf);
                bq.ascale = nullptr;
                launch_down_mm<QT_Q2B>(bq, nrec, s);
            } else {
                launch_down_mm<QT_T1>(bq, nrec, s);
            }
            continue;
        }
        d.items = items + (size_t)(q - 1) * L.maxrec;
        d.wl_len = flags + 8 + q;
        d.counters = flags + counter_set(1, q);
        if (q == QT_Q2B)
            launch_down_t<QT_Q2B>(d, nrec, s);
        else
            launch_down_t<QT_T1>(d, nrec, s);
    }
    mark(4);
    launch_combine(ys, CombineW{r.w, r.shared >= 0 ? r.gate : nullptr, r.res, r.kin}, out, T, kk, s);
    mark(5);
    return hip_status();
}

}  // namespace

extern "C" {

size_t rl_moe_workspace_bytes(int32_t T_max, int32_t k, int32_t E, int32_t H, int32_t I) {
    if (!shape_ok(T_max, k, E, H, I)) return 0;
    return layout(T_max, k, E, H, I).total;
}

int rl_moe_prefill(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, const rl_expert_blobs* experts,
                   float* out, int32_t T, int32_t k, void* workspace, size_t ws_bytes, void* stream) {
    return prefill_impl(x, routed_only(topk_ids, topk_w, k), experts, out, T, workspace, ws_bytes, stream, nullptr);
}

int rl_moe_prefill_block(const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                         const rl_expert_blobs* experts, int32_t shared_expert, const float* shared_gate,
                         const float* residual, float* out, int32_t T, int32_t k, void* workspace, size_t ws_bytes,
                         void* stream) {
    if (shared_expert < 0) return RL_EINVAL;
    const Route r{topk_ids, topk_w, k, shared_expert, shared_gate, residual};
    return prefill_impl(x, r, experts, out, T, workspace, ws_bytes, stream, nullptr);
}

int rl_moe_prefill_from_logits(const uint16_t* x, const float* logits, int32_t n_route, const rl_expert_blobs* experts,
                               int32_t shared_expert, const float* shared_gate, const float* residual, float* out,
                               int32_t* topk_ids, float* topk_w, int32_t T, int32_t k, void* workspace,
                               size_t ws_bytes, void* stream) {
    if (k < 1) return RL_ESHAPE;
    if (T > 0 && !logits) return RL_EINVAL;
    Route r{topk_ids, topk_w, k, shared_expert < 0 ? -1 : shared_expert, shared_gate, residual};
    r.logits = logits;
    r.n_route = n_route;
    return prefill_impl(x, r, experts, out, T, workspace, ws_bytes, stream, nullptr);
}

int rl_moe_prefill_noalloc(const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                           const rl_expert_blobs* experts, float* out, int32_t T, int32_t k, void* stream) {
    int present[3] = {0, 0, 0};
    const Route r = routed_only(topk_ids, topk_w, k);
    int rc = check_args(x, r, experts, out, T, present);
    if (rc != RL_OK || T == 0) return rc;
    if (layout(T, k, experts->E, experts->H, experts->I).total > RL_NOALLOC_SCRATCH_BYTES) return RL_ETOOBIG;
    void* ws = noalloc_scratch(true);
    if (ws == nullptr) return RL_EHIP;
    return prefill_impl(x, r, experts, out, T, ws, RL_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int rl_moe_noalloc_status(int32_t* flags_out) {
    if (!flags_out) return RL_EINVAL;
    void* ws = noalloc_scratch(false);
    if (ws == nullptr) return RL_EHIP;
    return rl_moe_status(ws, flags_out);
}

int rl_moe_prefill_timed(const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                         const rl_expert_blobs* experts, float* out, int32_t T, int32_t k, void* workspace,
                         size_t ws_bytes, void* stream, void* const* events) {
    if (!events) return RL_EINVAL;
    for (int i = 0; i < RL_TIMED_EVENTS; ++i)
        if (!events[i]) return RL_EINVAL;
    return prefill_impl(x, routed_only(topk_ids, topk_w, k), experts, out, T, workspace, ws_bytes, stream, events);
}

int rl_moe_gate_up(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, const rl_expert_blobs* experts,
                   uint16_t* h16_out, uint8_t* h8_out, uint32_t* hsc_out, int32_t T, int32_t k, void* workspace,
                   size_t ws_bytes, void* stream) {
    int present[3] = {0, 0, 0};
    const Route r = routed_only(topk_ids, topk_w, k);
    // validated with a stand-in for `out` (the hook has no layer output); the h buffers below
    int rc = check_args(x, r, experts, x, T, present);
    if (rc != RL_OK || T == 0) return rc;
    const bool split = t1_splits_h(present, experts->I);
    const bool need16 = present[QT_Q2B] > 0 || (present[QT_T1] > 0 && !split);
    if (need16 && (!h16_out || ((uintptr_t)h16_out & 1))) return RL_EINVAL;
    if (split && (!h8_out || !hsc_out || ((uintptr_t)hsc_out & 3))) return RL_EINVAL;
    rc = check_ws(experts, T, k, workspace, ws_bytes);
    if (rc != RL_OK) return rc;
    Layout L;
    run_group_gateup(x, r, experts, T, workspace, present, h16_out, static_cast<hipStream_t>(stream), L, nullptr,
                     split ? h8_out : nullptr, split ? hsc_out : nullptr);
    return hip_status();
}

static int decode_impl(const uint16_t* x, const Route& r, const rl_expert_blobs* experts, float* out, int32_t T,
                       void* workspace, size_t ws_bytes, void* stream) {
    int present[3] = {0, 0, 0};
    if (experts && (T < 1 || T > 2 || !gv_dim_ok(experts->H, 8) || !gv_dim_ok(experts->I, 4))) return RL_ESHAPE;
    int rc = check_layer(x, r, experts, out, T, workspace, ws_bytes, present);
    if (rc != RL_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int kk = r.kk();
    Layout L = layout(T, kk, experts->E, experts->H, experts->I);
    GvArgs a;
    a.x = x;
    a.pid = r.pid();
    a.w = r.w;
    a.gate = r.gate;
    a.res = r.res;
    a.arena = static_cast<const uint8_t*>(experts->arena);
    a.desc = experts->desc;
    a.hgv = at<uint16_t>(workspace, L.hbuf);  // [R*k][I] fp16
    a.pairs = at<GvPair>(workspace, L.gvpairs);
    a.out = out;
    a.flags = at<int32_t>(workspace, L.flags);
    a.R = T;
    a.k = kk;
    a.E = experts->E;
    a.H = experts->H;
    a.I = experts->I;
    const int mask = (present[QT_Q2B] ? 1 : 0) | (present[QT_T1] ? 2 : 0);
    if (mask == 1)
        launch_gv<1>(a, s);
    else if (mask == 2)
        launch_gv<2>(a, s);
    else
        launch_gv<3>(a, s);
    return hip_status();
}

int rl_moe_decode(const uint16_t* x, const int32_t* topk_ids, const float* topk_w, const rl_expert_blobs* experts,
                  float* out, int32_t T, int32_t k, void* workspace, size_t ws_bytes, void* stream) {
    return decode_impl(x, routed_only(topk_ids, topk_w, k), experts, out, T, workspace, ws_bytes, stream);
}

int rl_moe_decode_block(const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                        const rl_expert_blobs* experts, int32_t shared_expert, const float* shared_gate,
                        const float* residual, float* out, int32_t T, int32_t k, void* workspace, size_t ws_bytes,
                        void* stream) {
    if (shared_expert < 0) return RL_EINVAL;
    const Route r{topk_ids, topk_w, k, shared_expert, shared_gate, residual};
    return decode_impl(x, r, experts, out, T, workspace, ws_bytes, stream);
}

int rl_moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids, float* topk_w,
                 void* stream) {
    if (T < 0 || E < 1 || E > MAX_E || k < 1 || k > 16 || k > E) return RL_ESHAPE;
    if (T == 0) return RL_OK;
    if (!logits || !topk_ids || !topk_w) return RL_EINVAL;
    if (((uintptr_t)logits | (uintptr_t)topk_ids | (uintptr_t)topk_w) & 3) return RL_EINVAL;
    launch_route(logits, T, E, k, topk_ids, topk_w, static_cast<hipStream_t>(stream));
    return hip_status();
}

int rl_moe_group_pairs(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* offsets, int32_t* pair_src,
                       int32_t* inv, void* workspace, size_t ws_bytes, void* stream) {
    if (T < 0 || k < 1 || k > 16 || E < 1 || E > MAX_E || (int64_t)T * k > (1 << 24)) return RL_ESHAPE;
    if (!offsets || (T > 0 && (!topk_ids || !pair_src || !inv))) return RL_EINVAL;
    if (!workspace || ((uintptr_t)workspace % ALIGN)) return RL_EWORKSPACE;
    const Layout L = layout(T, k, E, 256, 64);
    if (ws_bytes < L.tile_hist + (size_t)tile_hist_rows((int64_t)T * k) * E * 4) return RL_EWORKSPACE;
    launch_group(PairIds{topk_ids, k, k, -1}, T, E, nullptr, offsets, pair_src, inv, at<int32_t>(workspace, L.flags),
                 at<int32_t>(workspace, L.tile_hist), nullptr, 0, static_cast<hipStream_t>(stream));
    return hip_status();
}

int rl_moe_dequant(int32_t qtype, int32_t decoder, const void* blocks, int64_t n_values, float* out, void* stream) {
    if (qtype != QT_Q2B && qtype != QT_T1) return RL_EINVAL;
    if (decoder < RL_DEC_STRIP || decoder > RL_DEC_ROWS_DOWN) return RL_EINVAL;
    if (n_values < 0 || n_values % 256) return RL_ESHAPE;
    if (n_values == 0) return RL_OK;
    if (!blocks || !out) return RL_EINVAL;
    const int64_t n_blocks = n_values / 256;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t* b = static_cast<const uint8_t*>(blocks);
    if (decoder == RL_DEC_STRIP) {
        dim3 grid((unsigned)((n_blocks * 4 + 255) / 256));
        if (qtype == QT_Q2B)
            hipLaunchKernelGGL(k_dequant<QT_Q2B>, grid, dim3(256), 0, s, b, n_blocks, out);
        else
            hipLaunchKernelGGL(k_dequant<QT_T1>, grid, dim3(256), 0, s, b, n_blocks, out);
        return hip_status();
    }
    if (decoder == RL_DEC_ROWS_GATEUP || decoder == RL_DEC_ROWS_DOWN) {
        dim3 grid((unsigned)((n_blocks * 16 + 255) / 256));
        const bool f16 = decoder == RL_DEC_ROWS_DOWN;
        if (qtype == QT_Q2B && !f16)
            hipLaunchKernelGGL((k_dequant_rows<QT_Q2B, false>), grid, dim3(256), 0, s, b, n_blocks, out);
        else if (qtype == QT_Q2B)
            hipLaunchKernelGGL((k_dequant_rows<QT_Q2B, true>), grid, dim3(256), 0, s, b, n_blocks, out);
        else if (!f16)
            hipLaunchKernelGGL((k_dequant_rows<QT_T1, false>), grid, dim3(256), 0, s, b, n_blocks, out);
        else
            hipLaunchKernelGGL((k_dequant_rows<QT_T1, true>), grid, dim3(256), 0, s, b, n_blocks, out);
        return hip_status();
    }
    // the blocks' bytes must be addressable by 32-bit buffer offsets from their dword base
    const uint32_t mis = (uint32_t)((uintptr_t)b & 3u);
    if ((uint64_t)mis + (uint64_t)n_blocks * (qtype == QT_T1 ? Fmt<QT_T1>::BYTES : Fmt<QT_Q2B>::BYTES) >
        0xFFFFFFF0ull)
        return RL_ESHAPE;
    const uint8_t* b4 = b - mis;
    dim3 grid((unsigned)((n_blocks + 63) / 64));  // 4 waves x 16 blocks per work-group
    if (qtype == QT_T1)
        hipLaunchKernelGGL((k_dequant_mfma<QT_T1, false>), grid, dim3(256), 0, s, b4, mis, n_blocks, out);
    else if (decoder == RL_DEC_MFMA_GATEUP)
        hipLaunchKernelGGL((k_dequant_mfma<QT_Q2B, false>), grid, dim3(256), 0, s, b4, mis, n_blocks, out);
    else
        hipLaunchKernelGGL((k_dequant_mfma<QT_Q2B, true>), grid, dim3(256), 0, s, b4, mis, n_blocks, out);
    return hip_status();
}

int rl_moe_status(const void* workspace, int32_t* flags_out) {
    if (!workspace || !flags_out) return RL_EINVAL;
    return hipMemcpy(flags_out, workspace, 4 * sizeof(int32_t), hipMemcpyDeviceToHost) == hipSuccess ? RL_OK
                                                                                                     : RL_EHIP;
}

const char* rl_moe_strerror(int status) {
    switch (status) {
        case RL_OK: return "ok";
        case RL_EINVAL: return "invalid argument (NULL pointer or unknown code)";
        case RL_ESHAPE: return "size outside the supported set";
        case RL_EWORKSPACE: return "workspace missing, misaligned or too small";
        case RL_EHIP: return "HIP runtime error at launch";
        case RL_EQTYPE: return "unknown block type in the expert descriptors";
        case RL_ETOOBIG: return "the call needs more than a fixed-size resource holds (no-allocation scratch, cache slots)";
        default: return "unknown status";
    }
}

}  // extern "C"
