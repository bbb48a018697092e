// HIP kernels of the routed-expert MoE layer for gfx950 (wave64).
//
//   k_count_split    pair histograms per tile of the grouping, and (other work-groups of the same
//                    launch) the split of x into hi/lo fp8 rows for the T1 experts
//   k_group_count    the pair histograms alone (layers without T1 experts, the grouping hook)
//   k_group_scatter  stable placement of the pairs by expert, offsets, per-type work lists
//   k_t1_f8          T1 experts on the fp8 MFMA (16x16x128): gate/up + SwiGLU -> h, for I <= 512
//                    already split into hi/lo fp8 rows for k_t1_dn, else fp16; also down for
//                    I > 512 (streamed split-h activations)
//   k_q2_mm          Q2B experts on the 16-bit MFMA (16x16x32), same structure: gate/up on bf16 x,
//                    down for I > 512 on fp16 h
//   k_split          split of fp16 h into hi/lo fp8 rows for the T1 down kernel when I > 512
//   k_t1_dn          T1 down for I <= 512, a chunk's split h rows held in LDS -> y slots
//   k_q2_dn          Q2B down for I <= 512, a chunk's fp16 h rows held in LDS -> y slots
//   k_down           both types with I < 256: decode + down on fp16 MFMA -> y slots
//                    (y: fp16 under a power-of-two scale per pair and 64 columns, y_store)
//   k_combine        out_t = sum_j w[t][j] * y_{t,j}, j ascending (selection order)
//   k_gv_gateup      1-2 row matrix-vector gate/up + SwiGLU (packed bf16 dot products)
//   k_gv_down        1-2 row matrix-vector down + ordered combine in one dispatch
//   k_dequant        block decode to fp32 through the same fragment decoder
// (The router, the step before the layer, is k_route in rl_route.h.)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rl_decode.h"
#include "rl_moe.h"

namespace rl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int FLAG_BAD_ID = 1;
constexpr int FLAG_BAD_QTYPE = 2;
constexpr int FLAGS_WORDS = 64;   // flags[0] error bits; flags[8 + q] work-list length of type q
constexpr int MAX_E = 1024;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// ---------------------------------------------------------------------------------------
// Pair grouping: two kernels over tiles of GT consecutive flattened pairs p = t*k + j.
//   k_group_count    per-tile expert histograms (and the clearing of the status words);
//   k_group_scatter  per tile: the pairs of expert e in earlier tiles (sum of their
//                    histograms) plus the exclusive scan of all counts place the tile's pairs;
//                    inside the tile wave w owns a contiguous run and lanes holding the same
//                    expert are found with ballots over the bits of the id and ranked by lane.
// The sorted order is (expert, token, slot), identical to a sequential stable sort.  One extra
// work-group (index ntiles, no pairs of its own) writes the offsets and the per-type work lists
// (experts with pairs, more pairs first; ties and experts above 255 pairs come in no particular
// order: the lists only steer scheduling) while the tiles scatter.
constexpr int GT = 1024;           // pairs per tile
constexpr int GROUP_NTHR = 256;    // threads per grouping work-group
constexpr int NBIN = 256;

// Work-list record of one expert: its pairs [p0, p0 + ne) in sorted order and the arena byte
// offsets of its gate, up and down matrices (32 bytes: one scalar load).
struct ItemRec {
    int32_t p0, ne;
    uint64_t off[3];
};

// Pairs of a call: token t, selection j < kk.  Selections j < kin are the caller's topk_ids
// (row stride kin); with a shared expert (shared >= 0) the last selection of every token is that
// expert, so the shared expert's pairs run through the same grouping, GEMMs and ordered combine.
struct PairIds {
    const int32_t* ids;  // [T][kin]
    int kin, kk, shared;
    __device__ __forceinline__ int expert(int p) const {
        if (shared < 0) return ids[p];
        const int t = p / kk, j = p - t * kk;
        return j < kin ? ids[t * kin + j] : shared;
    }
};

// Work records: an expert's sorted pairs in records of REC_PAIRS, except that an expert far above
// the layer's mean (more than REC_PAIRS pairs and more than 4x P / E: the shared expert has a
// pair for every token) is cut into records of REC_HOT, so that it is spread over many work items
// of about the size of the others.  96 pairs = two down chunks of 48 (or a 64-row and a 32-row
// gate/up chunk): no chunk of the down kernel is cut short by a record boundary (records of 64
// pairs made a 74-pair expert three down chunks, 48 + 16 + 10, and the Zipf-routed Q2B layer's
// down 17 us slower).  Records of 48 decode the weights as often as records of 96 do (one 48-row
// chunk each, against 64 + 32 rows) in items half as long: the MoE block of the 2048-token T1
// layer, whose shared expert has 2,048 pairs, ~19 us shorter; but where every expert has some
// hundreds of pairs (one GPU's share of experts), the 64-row gate/up chunks of 96-pair records
// are ~6 us faster.
constexpr int REC_PAIRS = 96;
constexpr int REC_HOT = REC_PAIRS / 2;
__host__ __device__ constexpr int rec_size(int pairs, int P, int E) {
    return pairs > REC_PAIRS && (int64_t)pairs * E > 4 * (int64_t)P ? REC_HOT : REC_PAIRS;
}
__host__ __device__ constexpr int max_records(int E, int P) { return E + (P + REC_HOT - 1) / REC_HOT; }

struct GroupArgs {
    PairIds pid;
    const rl_expert_desc* desc;  // may be NULL: no work lists
    int32_t* offsets;
    int32_t* pair_src;
    int32_t* inv;
    int32_t* flags;
    ItemRec* items;     // [2][maxrec]: per block type, records longest first
    int maxrec;
    int32_t* tile_hist; // [ntiles][E]
    int tp;             // pairs per tile (at most GT)
    u32x4* zero;        // the y scale bytes of the call, cleared by the first launch (may be NULL)
    int nzero;          // 16-byte words
    int P, E, ntiles;
    int nflags;         // status words to clear
};

// cleared by every work-group of the grouping's first launch (which precedes the down kernels)
__device__ __forceinline__ void clear_words(const GroupArgs& a) {
    for (int i = blockIdx.x * GROUP_NTHR + threadIdx.x; i < a.nzero; i += gridDim.x * GROUP_NTHR)
        a.zero[i] = u32x4{0u, 0u, 0u, 0u};
}

__device__ __forceinline__ void group_count_tile(const GroupArgs& a, int tile) {
    __shared__ int32_t h[MAX_E];
    const int tid = threadIdx.x;
    if (tile == 0 && tid < a.nflags) a.flags[tid] = 0;
    for (int e = tid; e < a.E; e += GROUP_NTHR) h[e] = 0;
    __syncthreads();
    const int p0 = tile * a.tp, p1 = min(a.P, p0 + a.tp);
    for (int p = p0 + tid; p < p1; p += GROUP_NTHR) {
        const int e = a.pid.expert(p);
        if (e >= 0 && e < a.E) atomicAdd(&h[e], 1);
    }
    __syncthreads();
    for (int e = tid; e < a.E; e += GROUP_NTHR) a.tile_hist[(size_t)tile * a.E + e] = h[e];
}

__global__ __launch_bounds__(GROUP_NTHR) void k_group_count(GroupArgs a) {
    clear_words(a);
    group_count_tile(a, blockIdx.x);
}

__global__ __launch_bounds__(GROUP_NTHR) void k_group_scatter(GroupArgs a) {
    constexpr int NW = GROUP_NTHR / 64;
    constexpr int SUB = GT / NW;
    __shared__ int32_t ids_sh[GT];
    __shared__ int32_t before[MAX_E];  // pairs of e in earlier tiles
    __shared__ int32_t tot[MAX_E];
    __shared__ int32_t scan[MAX_E];
    __shared__ int32_t whist[NW][MAX_E];
    __shared__ int32_t bins[2][NBIN];
    __shared__ int32_t wsum[NW];
    __shared__ int32_t bad_sh;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, tile = blockIdx.x;
    const bool lister = tile == a.ntiles;  // the offsets and work lists; no pairs (n <= 0)
    const int E = a.E;
    const int p0 = tile * a.tp, n = min(a.P - p0, a.tp);
    // the work-list builder's expert descriptors (e = tid + GROUP_NTHR * i), loaded before the
    // scans so that their latency overlaps them
    constexpr int EPL = MAX_E / GROUP_NTHR;
    rl_expert_desc dl[EPL];
    if (lister && a.desc != nullptr) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = tid + GROUP_NTHR * i;
            if (e < E) dl[i] = a.desc[e];
        }
    }
    if (tid == 0) bad_sh = 0;
    for (int i = tid; i < GT; i += GROUP_NTHR) ids_sh[i] = i < n ? a.pid.expert(p0 + i) : -1;
    {
        // pairs of each expert in earlier tiles and in all tiles; the histogram loads are issued
        // HB tiles at a time so that their latencies overlap
        constexpr int EPT = MAX_E / GROUP_NTHR;
        constexpr int HB = 8;
        int b[EPT], t[EPT];
#pragma unroll
        for (int i = 0; i < EPT; ++i) b[i] = t[i] = 0;
        for (int tl0 = 0; tl0 < a.ntiles; tl0 += HB) {
            int c[EPT][HB];
#pragma unroll
            for (int i = 0; i < EPT; ++i) {
                const int e = tid + GROUP_NTHR * i;
#pragma unroll
                for (int u = 0; u < HB; ++u)
                    c[i][u] = (e < E && tl0 + u < a.ntiles) ? a.tile_hist[(size_t)(tl0 + u) * E + e] : 0;
            }
#pragma unroll
            for (int i = 0; i < EPT; ++i)
#pragma unroll
                for (int u = 0; u < HB; ++u) {
                    b[i] += tl0 + u < tile ? c[i][u] : 0;
                    t[i] += c[i][u];
                }
        }
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid + GROUP_NTHR * i;
            before[e] = b[i];
            tot[e] = t[i];
        }
    }
    for (int i = tid; i < NW * MAX_E; i += GROUP_NTHR) (&whist[0][0])[i] = 0;
    __syncthreads();
    // inclusive scan of the totals: thread tid owns entries 4*tid .. 4*tid+3, a shuffle scan over
    // the lanes of each wave, then the sums of the waves before (one barrier)
    {
        static_assert(MAX_E == 4 * GROUP_NTHR, "four scan entries per thread");
        const int b = 4 * tid;
        const int s0 = tot[b], s1 = s0 + tot[b + 1], s2 = s1 + tot[b + 2], s3 = s2 + tot[b + 3];
        int incl = s3;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int ex = incl - s3;
        for (int w = 0; w < wave; ++w) ex += wsum[w];
        scan[b] = ex + s0;
        scan[b + 1] = ex + s1;
        scan[b + 2] = ex + s2;
        scan[b + 3] = ex + s3;
    }
    // wave-local counts of the tile
    const int r_begin = wave * SUB, r_end = min(r_begin + SUB, n);
    int bad = 0;
    for (int i = r_begin + lane; i < r_end; i += 64) {
        const int e = ids_sh[i];
        if (e >= 0 && e < E)
            atomicAdd(&whist[wave][e], 1);
        else
            bad = 1;
    }
    if (bad) atomicOr(&bad_sh, 1);
    __syncthreads();
    for (int e = tid; e < E; e += GROUP_NTHR) {
        int run = scan[e] - tot[e] + before[e];  // exclusive offset of e + pairs of e in earlier tiles
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int c = whist[w][e];
            whist[w][e] = run;
            run += c;
        }
    }
    if (lister)
        for (int e = tid; e <= E; e += GROUP_NTHR) a.offsets[e] = e == 0 ? 0 : scan[e - 1];
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int i0 = r_begin; i0 < r_end; i0 += 64) {
        const int i = i0 + lane;
        const int e = i < r_end ? ids_sh[i] : -1;
        const bool ok = (e >= 0 && e < E);
        uint64_t peers = __ballot(ok);
        for (int bit = 0; bit < 10; ++bit) {
            const uint64_t m = __ballot(ok && ((e >> bit) & 1));
            peers &= ((e >> bit) & 1) ? m : ~m;
        }
        if (ok) {
            const int pos = whist[wave][e] + __popcll(peers & lt_mask);
            a.pair_src[pos] = p0 + i;
            a.inv[p0 + i] = pos;
        } else if (i < r_end) {
            a.inv[p0 + i] = -1;
        }
        // every lane's read of whist[wave][e] happens before the leaders' updates, and the
        // updates before the next round's reads: LDS waits only (the pair_src / inv stores above
        // need not complete here)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
        if (ok && (peers & lt_mask) == 0) whist[wave][e] += __popcll(peers);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    if (tid == 0 && bad_sh) atomicOr(&a.flags[0], FLAG_BAD_ID);

    // per-type work lists of records (rec_size pairs at most), binned by record size,
    // larger records first
    if (lister && a.desc != nullptr) {
        static_assert(REC_PAIRS < NBIN, "record sizes are bins");
        for (int i = tid; i < 2 * NBIN; i += GROUP_NTHR) (&bins[0][0])[i] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = tid + GROUP_NTHR * i;
            if (e >= E) continue;
            const int q = dl[i].qtype, c = tot[e];
            if (c == 0) continue;
            if (q != QT_Q2B && q != QT_T1) {
                atomicOr(&bad_sh, 2);
                continue;
            }
            const int rp = rec_size(c, a.P, E);
            if (c >= rp) atomicAdd(&bins[q - 1][rp], c / rp);
            if (c % rp) atomicAdd(&bins[q - 1][c % rp], 1);
        }
        __syncthreads();
        if (tid < 128) {  // start of each bin in the type's list, high counts first: wave q scans type q
            static_assert(NBIN == 4 * 64, "four bins per lane");
            const int q = tid >> 6, l = tid & 63;
            int c[4], run = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // lane l owns bins 255-4l .. 252-4l (descending)
                c[j] = bins[q][NBIN - 1 - 4 * l - j];
                run += c[j];
            }
            int incl = run;  // inclusive scan over the lanes
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int v = __shfl_up(incl, d, 64);
                if (l >= d) incl += v;
            }
            int pos = incl - run;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bins[q][NBIN - 1 - 4 * l - j] = pos;
                pos += c[j];
            }
            if (l == 63) a.flags[8 + QT_Q2B + q] = incl;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = tid + GROUP_NTHR * i;
            if (e >= E) continue;
            const int q = dl[i].qtype, c = tot[e];
            if (c == 0 || (q != QT_Q2B && q != QT_T1)) continue;
            ItemRec r;
            r.off[0] = dl[i].gate_off;
            r.off[1] = dl[i].up_off;
            r.off[2] = dl[i].down_off;
            const int first = scan[e] - c;
            const int rp = rec_size(c, a.P, E);
            for (int p = 0; p < c; p += rp) {
                const int sz = min(rp, c - p);
                r.p0 = first + p;
                r.ne = sz;
                a.items[(size_t)(q - 1) * a.maxrec + atomicAdd(&bins[q - 1][sz], 1)] = r;
            }
        }
        __syncthreads();
        if (tid == 0 && (bad_sh & 2)) atomicOr(&a.flags[0], FLAG_BAD_QTYPE);
    }
}

// ---------------------------------------------------------------------------------------
// Scheduling of the expert GEMMs.  Work item = (expert rank, column slice); ranks come from the
// per-type work list, longest expert first.  Work-groups are dispatched round-robin over the 8
// XCDs, so blockIdx % 8 is the XCD; every XCD owns the ranks r = xcd (mod 8) and hands them out
// in order through its own counter (zeroed by the grouping's first launch), so all slices of one expert run on the
// same XCD (its gathered activation rows are read through one L2) and the XCD's work-groups
// balance themselves.
// flags[16 + 8*(2*stage + type - 1) + xcd]: per-XCD item counters, one set per stage and type
constexpr int CNT_BASE = 16;
__host__ __device__ constexpr int counter_set(int stage, int qtype) { return CNT_BASE + 8 * (2 * stage + qtype - 1); }

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uni64(uint64_t v) {
    return ((uint64_t)(uint32_t)uni((int)(v >> 32)) << 32) | (uint32_t)uni((int)(uint32_t)v);
}

__device__ __forceinline__ bool next_item(int32_t* counters, int ns, int n_ranks, int* sh, int& rank, int& slice) {
    const int xcd = blockIdx.x & 7;
    if (threadIdx.x == 0) *sh = atomicAdd(&counters[xcd], 1);
    __syncthreads();
    const int local = uni(*sh);  // the same for the whole work-group
    __syncthreads();
    rank = (local / ns) * 8 + xcd;
    slice = local % ns;
    return rank < n_ranks;
}

// Decode tables of one block type, built once per (persistent) work-group.
template <int QT, bool F16>
struct alignas(16) DecodeTables {
    uint64_t val[val_entries<QT>()];
    uint32_t tern[QT == QT_T1 ? 256 : 4];  // (Q2B: padding to whole 16-byte units)
    __device__ inline void build(int tid, int nthr) {
        for (int i = tid; i < val_entries<QT>(); i += nthr) val[i] = val_entry<QT, F16>(i);
        if constexpr (QT == QT_T1)
            for (int i = tid; i < 256; i += nthr) tern[i] = tern_entry((uint32_t)i);
    }
};

// The same tables as initialised device data (evaluated by the compiler from the same entry
// functions): short-lived work-groups copy them into LDS with 16-byte loads instead of computing
// them.
template <int QT, bool F16>
constexpr DecodeTables<QT, F16> make_tables() {
    DecodeTables<QT, F16> t{};
    for (int i = 0; i < val_entries<QT>(); ++i) t.val[i] = val_entry<QT, F16>(i);
    if constexpr (QT == QT_T1)
        for (int i = 0; i < 256; ++i) t.tern[i] = tern_entry((uint32_t)i);
    return t;
}
template <int QT, bool F16>
__device__ constexpr DecodeTables<QT, F16> kDecodeTables = make_tables<QT, F16>();

template <int QT, bool F16>
__device__ __forceinline__ void copy_tables(DecodeTables<QT, F16>& dst, int tid, int nthr) {
    static_assert(sizeof(DecodeTables<QT, F16>) % 16 == 0, "whole 16-byte units");
    constexpr int N = (int)(sizeof(DecodeTables<QT, F16>) / 16);
    const u32x4* s = reinterpret_cast<const u32x4*>(&kDecodeTables<QT, F16>);
    u32x4* d = reinterpret_cast<u32x4*>(&dst);
    for (int i = tid; i < N; i += nthr) d[i] = s[i];
}

__device__ __forceinline__ float silu_fast(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Running block scale: the accumulator holds sum_b (d_b / d_cur) * S_b, so each new block only
// rescales it by d_prev/d_cur and the MFMA adds the integer dot product S_b directly.  A block
// with d = 0 contributes nothing (its operands are zero, see Strip::prepare) and keeps the scale.
struct RunScale {
    float dprev = 1.0f;
    __device__ __forceinline__ float step(float d) {
        const float eff = d == 0.0f ? dprev : d;
        const float r = dprev * __builtin_amdgcn_rcpf(eff);
        dprev = eff;
        return r;
    }
};

// Activation chunk of the K loop: for each of the 4 lane groups, CS*8 consecutive k of its
// strip; staged as [64 rows][4 groups][CS*8] halfwords (+8 pad per row), 16-byte pieces.
template <int CS, int NTHR>
struct ChunkShape {
    static constexpr int SEG = CS * 8;          // k values per group per chunk
    static constexpr int LDA = 4 * SEG + 8;     // halfwords per staged row
    static constexpr int PIECES = 4 * SEG / 8;  // 16-byte pieces per row
    static constexpr int TOTAL = 64 * PIECES;   // pieces per chunk
    static constexpr int PER_THREAD = (TOTAL + NTHR - 1) / NTHR;
};

// Staging of one activation chunk by the NTHR threads of a work-group: thread tid owns pieces
// tid + NTHR*i (row = piece / PIECES); `off` are byte offsets of the pieces' sources (row,
// group, position) without the chunk's own k offset.
template <int CS, int NTHR>
struct Stager {
    using CH = ChunkShape<CS, NTHR>;
    uint32_t off[CH::PER_THREAD];
    u32x4 v[CH::PER_THREAD];
    __device__ __forceinline__ void load(const BufSrc& src, uint32_t koff, int tid) {
#pragma unroll
        for (int i = 0; i < CH::PER_THREAD; ++i)
            if (CH::TOTAL % NTHR == 0 || tid + NTHR * i < CH::TOTAL)
                v[i] = __builtin_amdgcn_raw_buffer_load_b128(src.r, off[i] + koff, 0, 0);
    }
    __device__ __forceinline__ void store(uint16_t* As, int tid) const {
#pragma unroll
        for (int i = 0; i < CH::PER_THREAD; ++i) {
            const int idx = tid + NTHR * i;
            if (CH::TOTAL % NTHR == 0 || idx < CH::TOTAL)
                *(u32x4*)&As[(idx / CH::PIECES) * CH::LDA + 8 * (idx % CH::PIECES)] = v[i];
        }
    }
};

// ---------------------------------------------------------------------------------------
// T1 gate/up on the fp8 MFMA (16x16x128).  T1 operands s*t (|s*t| <= 7) are exact in fp8
// e4m3; the decoder (T1Dec8) produces them with one LDS lookup per digit byte and one
// byte-select per four weights.  The bf16 activations become an exact pair hi + lo of fp8
// values after a per-token power-of-two scaling 2^sigma (max |x| * 2^sigma in [128, 256)):
// hi = fp8(v), lo = fp8(v - hi) keeps all 8 significant bits of v except for elements below
// ~2^-10 of the row's maximum.  Two fp8 MFMAs (hi, lo) take the same MFMA time as one bf16
// MFMA over the same k.

// Activation rows split into hi/lo fp8 in the decoder's k order: row r of K values (bf16 x or
// fp16 h) -> 2K bytes ordered [kb][h][g][hi 32 | lo 32], where byte p of the 32-byte group
// (kb, h, g) holds k = 256*kb + t1_kmap(g, 32*h + p).  Each row is scaled by 2^sigma (max |v| *
// 2^sigma in [128, 256)); hi = fp8(v), lo = fp8(v - hi).  The 32 values of a group are two
// contiguous runs of the row (60g + 32h .. and, for h = 1, the four tail values 240 + 4g ..), so
// one lane converts a whole group and writes its 64 bytes.  LPR lanes per row, NG groups per lane.
// scale[r] = 2^-sigma(r).  SPLIT_X: bf16 token rows (x); SPLIT_H: fp16 sorted-pair rows (h).
enum { SPLIT_X = 0, SPLIT_H = 1 };
struct SplitArgs {
    const uint16_t* src;
    uint8_t* dst;
    float* scale;  // [rows]
    int rows, K;
};

template <int MODE, int LPR, int NG>
__device__ __forceinline__ void split_rows(const SplitArgs& a, int blk) {
    constexpr int RPB = 256 / LPR;
    // the block's rows pass through LDS: coalesced 16-byte global loads, then 8-byte reads of
    // each group's two runs
    __shared__ __attribute__((aligned(16))) uint8_t stage[256 * 64 * NG];
    const int sub = threadIdx.x % LPR, rl = (int)threadIdx.x / LPR, r = blk * RPB + rl;
    const bool live = r < a.rows;
    const int G = a.K >> 5;
    const uint8_t* row = (const uint8_t*)(a.src + (size_t)(live ? r : 0) * a.K);
    uint8_t* srow = stage + rl * (64 * LPR * NG);
#pragma unroll
    for (int n = 0; n < NG; ++n) {
        const int gi = sub + LPR * n;
        if (gi < G) {
#pragma unroll
            for (int i = 0; i < 4; ++i) *(u32x4*)(srow + 64 * gi + 16 * i) = *(const u32x4*)(row + 64 * gi + 16 * i);
        }
    }
    __syncthreads();
    const uint16_t* lrow = (const uint16_t*)srow;
    uint2 raw[NG][8];
    float amax = 0.f;
#pragma unroll
    for (int n = 0; n < NG; ++n) {
        const int gi = sub + LPR * n;
        const int gl = gi < G ? gi : 0;
        const int kb = gl >> 3, hh = (gl >> 2) & 1, g = gl & 3;
        const int base = 256 * kb + 60 * g + 32 * hh;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int off = (hh == 0 || i < 7) ? base + 4 * i : 256 * kb + 240 + 4 * g;
            raw[n][i] = *(const uint2*)(lrow + off);
        }
        if (gi < G) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint32_t w = q ? raw[n][i].y : raw[n][i].x;
                    const float f0 = MODE == SPLIT_X ? __uint_as_float(w << 16) : half_bits_to_float(w & 0xFFFFu);
                    const float f1 = MODE == SPLIT_X ? __uint_as_float(w & 0xFFFF0000u) : half_bits_to_float(w >> 16);
                    amax = fmaxf(amax, fmaxf(fabsf(f0), fabsf(f1)));
                }
            }
        }
    }
#pragma unroll
    for (int d = LPR / 2; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    const int ex = amax > 0.f ? (int)((__float_as_uint(amax) >> 23) & 255u) - 127 : 7;  // floor(log2(amax))
    int sigma = 7 - ex;
    sigma = sigma < -120 ? -120 : (sigma > 120 ? 120 : sigma);
    const float sc = __uint_as_float((uint32_t)(127 + sigma) << 23);
    const float inv_sc = __uint_as_float((uint32_t)(127 - sigma) << 23);
    if (!live) return;
    uint8_t* drow = a.dst + (size_t)r * 2 * a.K;
#pragma unroll
    for (int n = 0; n < NG; ++n) {
        const int gi = sub + LPR * n;
        if (gi >= G) continue;
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float x[4];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const uint32_t w = q ? raw[n][i].y : raw[n][i].x;
                x[2 * q] = (MODE == SPLIT_X ? __uint_as_float(w << 16) : half_bits_to_float(w & 0xFFFFu)) * sc;
                x[2 * q + 1] = (MODE == SPLIT_X ? __uint_as_float(w & 0xFFFF0000u) : half_bits_to_float(w >> 16)) * sc;
            }
            uint32_t h = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
            h = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], (int)h, true);
            uint32_t l = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[0] - __builtin_amdgcn_cvt_f32_fp8((int)h, 0),
                                                                   x[1] - __builtin_amdgcn_cvt_f32_fp8((int)h, 1), 0, false);
            l = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[2] - __builtin_amdgcn_cvt_f32_fp8((int)h, 2),
                                                          x[3] - __builtin_amdgcn_cvt_f32_fp8((int)h, 3), (int)l, true);
            hi[i] = h;
            lo[i] = l;
        }
        u32x4* out = (u32x4*)(drow + 64 * gi);
        out[0] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        out[1] = u32x4{hi[4], hi[5], hi[6], hi[7]};
        out[2] = u32x4{lo[0], lo[1], lo[2], lo[3]};
        out[3] = u32x4{lo[4], lo[5], lo[6], lo[7]};
    }
    if (sub == 0) a.scale[r] = inv_sc;
}

template <int MODE, int LPR, int NG>
__global__ __launch_bounds__(256) void k_split(SplitArgs a) {
    split_rows<MODE, LPR, NG>(a, blockIdx.x);
}

// The pair histograms of the grouping and the split of x in one launch (they are independent):
// work-groups [0, ntiles) count, the others split 256/LPR token rows each.
template <int LPR, int NG>
__global__ __launch_bounds__(256) void k_count_split(GroupArgs g, SplitArgs a) {
    static_assert(GROUP_NTHR == 256, "one thread layout for both parts");
    clear_words(g);
    if ((int)blockIdx.x < g.ntiles)
        group_count_tile(g, blockIdx.x);
    else
        split_rows<SPLIT_X, LPR, NG>(a, blockIdx.x - g.ntiles);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// sa: this lane's E8M0 scale (2^(sa-127)) for A; B is unscaled.  As measured on gfx950, the
// scale of row i and 32-value k-block s comes from lane 16s + i, and block s is dwords
// 4*(s >> 1) .. +3 of lane groups 2*(s & 1) and 2*(s & 1) + 1.  The two halves of lane group g's
// operand are thus scaled by lane groups g >> 1 and 2 + (g >> 1), which lane groups g and g ^ 1
// share: lane group L supplies the scale of the k-group pair {2*(L & 1), 2*(L & 1) + 1}.
__device__ __forceinline__ f32x4 mfma_f8(const uint32_t* a, const uint32_t* b, f32x4 c, int sa) {
    i32x8 av, bv;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        av[i] = (int)a[i];
        bv[i] = (int)b[i];
    }
    // formats 0/0 = fp8 e4m3 for both operands; B's E8M0 scale is 1 (127)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, sa, 0, 127);
}

// 16x16x32 MFMA on 16-bit operands: fp16 (F16) or bf16; b holds the B operand's four dwords.
template <bool F16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, const uint32_t* b, f32x4 c) {
    const u32x4 bv = {b[0], b[1], b[2], b[3]};
    return F16 ? mfma_f16(a, bv, c) : mfma_bf16(a, bv, c);
}

// The expert GEMMs with weight windows and activations staged in LDS, one instance per block
// type: T1 on the fp8 MFMA (16x16x128; activations split into hi/lo e4m3 rows in t1_kmap order,
// one 2^-sigma scale per row), Q2B on the 16-bit MFMA (16x16x32; gate/up reads x as bf16 and down
// reads h as fp16, both as they are, rows in plain order).  Gate/up: activations gathered through
// the token pair_src[p] / k of each sorted pair p, weights gate and up [I][H], output h (fp16,
// SwiGLU, sorted-pair rows).  Down: activations in sorted-pair rows, weights down [H][I], output
// y (fp16, row = original pair index t*k + j).  K is the contracted length, N the output width.
// Per-pair outputs y of the down GEMMs, kept for the ordered combine (k_combine): fp16 under a
// power-of-two scale 2^sigma per (pair, 64-column tile).  sigma = 0 (fp16 as it is) unless a
// value of the storing wave reaches 2^15; then every tile of that wave takes the sigma that puts
// its own largest |y| in [2^14, 2^15), so no finite y overflows and each keeps fp16's 11
// significant bits relative to its tile maximum.  The sigma bytes are zeroed by the grouping's
// first launch and written only by the scaled stores.
constexpr int CT = 64;          // columns per scale tile
constexpr int Y_SPARE = 4096;   // waves of a down launch (each stores its padding rows apart)
struct YSlots {
    uint16_t* yslot;  // [P][H] fp16 bits, row t*k + j: y * 2^sigma
    int8_t* yexp;     // [P][H/CT] sigma of each (pair, tile)
    uint16_t* yspare; // [Y_SPARE][CT]: each wave's own target for its padding rows (never read)
    int8_t* espare;   // [Y_SPARE]
    int H, P;
};

enum { GU_GATEUP = 0, GU_DOWN = 1 };
struct GuArgs {
    const uint8_t* act;       // [rows][2K bytes] activations (see above)
    const float* ascale;      // T1: 2^-sigma of each activation row (gate/up: [T] per token; down: [P])
    const int32_t* pair_src;  // original pair index t*k + j of each sorted pair
    const uint8_t* arena;
    const ItemRec* items;     // this type's work list, longest first
    const int32_t* wl_len;    // its length (device)
    uint16_t* hbuf;           // gate/up output [P][N] fp16
    uint8_t* h8;              // T1 gate/up, I <= 512: h written here as hi/lo fp8 rows instead (null: hbuf)
    uint32_t* hsc;            // with h8, and read by the T1 down kernel: byte 2*kb + p of word r = E8M0
                              // scale of k-groups 2p, 2p+1 of block kb of h row r
    YSlots ys;                // down: the per-pair outputs
    int32_t* flags;           // status words (flags[0])
    int K, N, ns;
    int k;                    // pairs per token (gate/up: token of pair index q is q / k)
    int P;                    // pairs: the length of pair_src (down: y has a spare row P for padding rows)
};

// Work item of the gate/up kernel: GU_NW waves, each with NTI 16-column tiles of gate and the
// same NTI tiles of up (NT = 2*NTI weight strips per lane); an item covers 16*NTI*GU_NW columns
// of I for one 64-pair chunk at a time.  All operands reach LDS by direct buffer-to-LDS loads
// (no registers in flight):
//  - activations: a ring of 2 steps of 16 KB (two separate arrays, so that the compiler can
//    tell their loads apart), each step loaded one step ahead and shared by the work-group;
//  - weights: each wave loads the next block of its own rows into its own area, right after it
//    has read the current block out of it: WL consecutive lanes fetch one row's window (a
//    coalesced pattern; the lanes that decode a row are 16 apart, so loading into registers
//    directly would not coalesce).  A strip's 16 windows are written by four loads of 4*WL
//    active lanes (4 rows each) at WQ-byte spacing, which puts the rows that one LDS read
//    serves in distinct banks (a plain window-size spacing would put them in fewer).
// The waits on the shared ring are counted explicitly (vm_barrier).  Per wave, vector-memory
// instructions are issued in the fixed order
//   step 2kb: act(2kb+1) [GU_DMA], wts(kb+1) [4*NT] | step 2kb+1: act(2kb+2) [GU_DMA]
// (prologue: act(0), wts(0); in place of the last block's wts(nkb) and act(NS) a chunk loads the
// next chunk's wts(0) and act(0), and the next chunk then starts with a full wait only), so when
// step c waits for act(c) at most 0 (c even) or 4*NT (c odd) later loads may still be in
// flight, and no activation wait covers the windows.  A wave reads the windows of block kb at
// the top of the block, after waiting until at most GU_DMA of its loads (the activation step
// issued after those windows) are outstanding; the windows thus have two steps to land.  The
// compiler's own tracking of buffer-to-LDS loads is not relied on: it can miss them.
constexpr int GU_STEP = 64 * 256;  // one staged step: 64 rows x 256 bytes (128 values of k)
constexpr int GU_NW = 4;
constexpr int GU_DMA = GU_STEP / 1024 / GU_NW;  // 1 KB buffer-to-LDS loads per wave per step

// Weight-window geometry of a block type: WIN bytes per row window (the whole block, from the
// dword boundary at or below its start), fetched by WL lanes of 16 bytes each; a strip's 16
// windows sit in four quarters of 4 rows, WQ bytes apart.  WQ (a multiple of 16) is chosen so
// that the decoders' reads of the 16 rows of a strip spread over the LDS banks: T1 4 windows + 16
// bytes (a quarter of the conflicts of a plain 4-window spacing), Q2B 4 windows + 32 bytes (a
// third fewer than at + 16 bytes).
template <int QT>
struct WinGeo;
template <>
struct WinGeo<QT_T1> {
    static constexpr int WIN = 64, WL = 4, WQ = 4 * 64 + 16, WS = 4 * WQ;
};
template <>
struct WinGeo<QT_Q2B> {
    static constexpr int WIN = 80, WL = 5, WQ = 4 * 80 + 32, WS = 4 * WQ;
};
// for a fetching lane (< 4*WL): the row of its quarter it serves, and the byte offset of its 16
// bytes in that row's window
template <int QT>
__device__ __forceinline__ uint32_t win_lane_row(int lane) {
    return QT == QT_T1 ? (uint32_t)((lane >> 2) & 3) : (uint32_t)((lane / 5) & 3);
}
template <int QT>
__device__ __forceinline__ uint32_t win_lane_byte(int lane) {
    return QT == QT_T1 ? 16u * (uint32_t)(lane & 3) : 16u * (uint32_t)(lane % 5);
}

// LDS layout of one wave's windows of NT strips.  Narrow (the general case): per strip four
// quarters of 4 rows, WQ bytes apart, each quarter loaded by its own buffer-to-LDS instruction of
// 4*WL active lanes (4*NT instructions per block).  Wide (T1, 4 strips of one matrix: WL = 4, so
// 64 lanes cover one quarter of all four strips): quarter q holds [strip][row][64 bytes] followed
// by 16 bytes of padding, and lane L fetches 16 bytes (L & 3) of row 4q + ((L >> 2) & 3) of strip
// L >> 4, so one 64-lane instruction per quarter loads it (4 per block instead of 16: the down
// kernels 6.5 us faster).  Gate/up strips come from two matrices: the wide layout then needs one
// buffer resource spanning both (SPAN, 9 us faster; two resources, i.e. two 32-lane instructions
// per quarter, measured 10 us slower than the narrow layout).  In both layouts the 16 rows of a
// strip read by one lane group fall on distinct banks: wide row 4q + j of strip t starts at
// 1040q + 256t + 64j bytes, bank 4q + 16j.
// Linear (Q2B, 4 strips from one resource): the 64 rows' 80-byte windows back to back (row 16t +
// r at 80 (16t + r) bytes: 80 bytes = 20 banks, so 16 consecutive rows fall on distinct banks),
// filled by 5 instructions of 64 lanes (slot s = 64i + L holds 16 bytes s % 5 of row s / 5).
template <int QT, int NT, int NMAT, bool SPAN = true>
struct WinLay {
    typedef WinGeo<QT> G;
    static constexpr bool ONE_RES = NT == 4 && (NMAT == 1 || SPAN);
    static constexpr bool WIDE = QT == QT_T1 && ONE_RES;
    static constexpr bool LINEAR = QT == QT_Q2B && ONE_RES;
    static constexpr int QS = NT * 256 + 16;  // wide: bytes per quarter
    static constexpr int WAVE_BYTES = WIDE ? 4 * QS : LINEAR ? NT * 16 * G::WIN : NT * G::WS;
    // per-lane offsets per block (wide: one per quarter; linear: one per instruction; narrow: one per strip)
    static constexpr int NOFF = LINEAR ? NT * 16 * G::WIN / 1024 : NT;
    static constexpr int LOADS = WIDE ? 4 : LINEAR ? NOFF : 4 * NT;  // buffer-to-LDS instructions per block
    static_assert(!LINEAR || (NT * 16 * G::WIN) % 1024 == 0, "whole 64-lane loads");
    __device__ static __forceinline__ const uint32_t* win(uint8_t* wave_base, int t, int r) {
        if constexpr (WIDE)
            return (const uint32_t*)(wave_base + QS * (r >> 2) + 256 * t + 64 * (r & 3));
        else if constexpr (LINEAR)
            return (const uint32_t*)(wave_base + (16 * t + r) * G::WIN);
        else
            return (const uint32_t*)(wave_base + t * G::WS + G::WQ * (r >> 2) + G::WIN * (r & 3));
    }
    // one-resource layouts: the strip, row and 16-byte piece that `lane` fetches with load i, and
    // that load's LDS offset in the wave's area
    __device__ static __forceinline__ void lane_piece(int i, int lane, int& t, int& r, int& p) {
        if constexpr (WIDE) {
            t = lane >> 4;
            r = 4 * i + ((lane >> 2) & 3);
            p = lane & 3;
        } else {
            const int sl = 64 * i + lane, R = sl / 5;
            t = R >> 4;
            r = R & 15;
            p = sl - 5 * R;
        }
    }
    __device__ static __forceinline__ int load_lds_off(int i) { return WIDE ? QS * i : 1024 * i; }
};

// A staged step of an activation row is 256 bytes in 16 pieces of 16 bytes; piece 4g + j
// (lane group g, operand quarter j) sits at slot (4g + j) ^ (row % 16) of the row (spreading the
// rows that one LDS read serves over the banks), so the loading lane of slot s fetches piece
// s ^ (row % 16).  act_piece_off(P) is piece P's byte offset in the row relative to
// act_step_off(c), the offset of step c:
//   T1 (split rows, already in t1_kmap order): 256c + 16P;
//   Q2B (plain 16-bit rows): piece 4g + j of step c holds values 256(c/2) + 64g + 32(c%2) + 8j
//   .. +7 (q2_kmap), i.e. bytes 512(c/2) + 64(c%2) + 128g + 16j.
template <int QT>
__device__ __forceinline__ uint32_t act_piece_off(int P) {
    return QT == QT_T1 ? 16u * (uint32_t)P : 128u * (uint32_t)(P >> 2) + 16u * (uint32_t)(P & 3);
}
template <int QT>
__device__ __forceinline__ uint32_t act_step_off(int c) {
    return QT == QT_T1 ? (uint32_t)c * 256u : 512u * (uint32_t)(c >> 1) + 64u * (uint32_t)(c & 1);
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void mem_fence_compiler() { asm volatile("" ::: "memory"); }

// Wait until at most N vector-memory loads of this wave are outstanding and all its LDS reads
// are done, then synchronise the work-group.  One asm statement, so nothing is moved between
// the wait and the barrier, and no memory access moves across it.
template <int N>
__device__ __forceinline__ void vm_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Work-group barrier for LDS data only (no wait on outstanding global stores or loads).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct GuShared {
    uint8_t* ring[2];
    uint8_t* wts;  // [GU_NW][NT][WS]: per wave and strip, 16 row windows
    const uint64_t* tsel;   // T1 tables
    const uint32_t* tbl8;
    float* rscale;
    int32_t* rdst;
    const uint64_t* qsel;   // Q2B tables
    const uint64_t* q2row;
    float* hred;            // T1 gate/up: [GU_NW][64] per-wave row maxima of h
};

// Decoder tables of a block type in LDS (T1: digit selectors and fp8 scale tables; Q2B: code
// selectors and the 16-bit value rows, bf16 or fp16 after F16), built by the work-group.
template <int QT, bool F16>
struct GuTables {
    static constexpr int N64 = QT == QT_T1 ? TSEL_ENTRIES : QSEL_ENTRIES + Q2ROW_ENTRIES;
    __device__ static inline void build(uint64_t* t64, uint32_t* tbl8, int tid, int nthr) {
        if constexpr (QT == QT_T1) {
            for (int i = tid; i < TSEL_ENTRIES; i += nthr) t64[i] = tsel_entry(i);
            if (tid < 8) {  // [e(-s), e(0), e(+s), 0] with the hardware's fp8 encoding; s = 0 -> all zero
                const float sv = (float)tid;
                const uint32_t pos = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sv, 0.f, 0, false) & 255u;
                const uint32_t neg = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(-sv, 0.f, 0, false) & 255u;
                tbl8[tid] = tid == 0 ? 0u : (neg | (pos << 16));
            }
        } else {
            for (int i = tid; i < N64; i += nthr)
                t64[i] = i < QSEL_ENTRIES ? qsel_entry(i) : q2row_entry<F16>(i - QSEL_ENTRIES);
        }
    }
    __device__ static inline GuShared shared(uint8_t* r0, uint8_t* r1, uint8_t* wts, const uint64_t* t64,
                                             const uint32_t* tbl8, float* rscale, int32_t* rdst) {
        return GuShared{{r0, r1}, wts, t64, tbl8, rscale, rdst, t64, t64 + QSEL_ENTRIES};
    }
};

// Static schedule of one XCD's share of a type's work list: ranks r = xcd (mod 8), each cut
// into ns column slices, item ix -> (rank 8*(ix / ns) + xcd, slice ix % ns).  The nw
// work-groups of the XCD (blockIdx = 8*j + xcd: work-groups are dealt round-robin over the
// XCDs) take the items in snake order, round q taking item q*nw + j (q even) or
// q*nw + nw-1-j (q odd), which balances a longest-first list without atomics; every item of
// an expert stays on one XCD (one L2 for its activation rows).  HALVES: the first half of the
// XCD's work-groups (j < nw/2, one per CU) takes the first, longer half of every round and the
// second half the rest, each half in its own snake order.  The second work-group dispatched to
// a CU issues behind the first one's waves: per-work-group time stamps of the gate/up kernel put
// j < nw/2 at ~121 us and j >= nw/2 at ~137 us for the same work (a reversed assignment keeps
// the gap with the position, not the items); with the halves the kernel is 0.5-4 us shorter
// (the down kernel, whose halves differ less, gains nothing).
struct StaticSched {
    int xcd, j, nw, ns, nitems;
    bool halves;
    __device__ inline StaticSched(int n_ranks, int ns_, bool halves_ = false) {
        xcd = blockIdx.x & 7;
        j = blockIdx.x >> 3;
        nw = gridDim.x >> 3;
        ns = ns_;
        nitems = (n_ranks > xcd ? (n_ranks - xcd + 7) / 8 : 0) * ns;
        halves = halves_ && nw >= 2 && (nw & 1) == 0;
    }
    __device__ inline int item(int q) const {
        if (!halves) return q * nw + ((q & 1) ? nw - 1 - j : j);
        const int h = nw >> 1, m = j >= h ? 1 : 0, jj = j - m * h;
        return q * nw + m * h + ((q & 1) ? h - 1 - jj : jj);
    }
    __device__ inline int rank(int ix) const { return (ix / ns) * 8 + xcd; }
    __device__ inline int slice(int ix) const { return ix % ns; }
};

// scalar (uniform) load of a work-list record
__device__ __forceinline__ ItemRec load_item(const ItemRec* items, int rank) {
    typedef const __attribute__((address_space(4))) uint64_t* cptr;
    const cptr p = (cptr)(items + rank);
    const uint64_t w0 = p[0];
    ItemRec r;
    r.p0 = (int32_t)(uint32_t)w0;
    r.ne = (int32_t)(uint32_t)(w0 >> 32);
    r.off[0] = p[1];
    r.off[1] = p[2];
    r.off[2] = p[3];
    return r;
}

// Decoder of one strip: the T1 byte-strip decoder or the Q2B 16-bit one.
template <int QT>
struct StripDec;
template <>
struct StripDec<QT_T1> {
    typedef T1Dec8 type;
};
template <>
struct StripDec<QT_Q2B> {
    typedef Q2Dec16 type;
};

// decoder state of one strip from its row window (m = block start % 4)
template <int QT>
__device__ __forceinline__ void strip_prep(typename StripDec<QT>::type& dec, const uint32_t* win, uint32_t m, int g,
                                           const T1Lane8& ln, const GuShared& sh) {
    if constexpr (QT == QT_T1) {
        T1Raw8 raw;
        raw.load_window(win, m, g);
        dec.prep(raw, ln, sh.tbl8);
    } else {
        Q2Raw16 raw;
        raw.load_window(win, m, g);
        dec.prep(raw, sh.q2row);
    }
}

// The MFMAs of one staged step h for MT row tiles x NT strips (activation step in `ring`, rows
// of 256 bytes); F16 picks fp16 over bf16 operands on the 16-bit path.  T1: sa[mt] is the E8M0
// scale of the lane's activation values in row tile mt (127 = 1).
template <int QT, bool F16, int MT, int NT, int H>
__device__ __forceinline__ void step_mfma(const typename StripDec<QT>::type* dec, const T1Lane8& ln,
                                          const GuShared& sh, const uint8_t* ring, int m, int g, f32x4 (&acc)[MT][NT],
                                          const int (&sa)[MT]) {
    if constexpr (QT == QT_T1) {
        uint32_t b[NT][8];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            dec[t].step(H, ln, sh.tsel, b[t]);
            __builtin_amdgcn_sched_barrier(0);  // one strip's lookups in flight at a time
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint8_t* rp = ring + (mt * 16 + m) * 256;
            uint32_t ahi[8], alo[8];
            *(u32x4*)&ahi[0] = *(const u32x4*)(rp + (((4 * g + 0) ^ m) << 4));
            *(u32x4*)&ahi[4] = *(const u32x4*)(rp + (((4 * g + 1) ^ m) << 4));
            *(u32x4*)&alo[0] = *(const u32x4*)(rp + (((4 * g + 2) ^ m) << 4));
            *(u32x4*)&alo[4] = *(const u32x4*)(rp + (((4 * g + 3) ^ m) << 4));
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                acc[mt][t] = mfma_f8(ahi, b[t], acc[mt][t], sa[mt]);
                acc[mt][t] = mfma_f8(alo, b[t], acc[mt][t], sa[mt]);
            }
            __builtin_amdgcn_sched_barrier(0);  // one M tile's activation operands at a time
        }
    } else {
        // two halves of two 16x16x32 MFMAs each (operands 2p, 2p+1: one sub-scale)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            uint32_t b[NT][8];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                dec[t].half(H, p, sh.qsel, b[t]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint8_t* rp = ring + (mt * 16 + m) * 256;
                const u32x4 a0 = *(const u32x4*)(rp + (((4 * g + 2 * p) ^ m) << 4));
                const u32x4 a1 = *(const u32x4*)(rp + (((4 * g + 2 * p + 1) ^ m) << 4));
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    acc[mt][t] = mfma16<F16>(a0, &b[t][0], acc[mt][t]);
                    acc[mt][t] = mfma16<F16>(a1, &b[t][4], acc[mt][t]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// Output column order of the T1 gate/up kernel: position q = 256*kb + 64*g + j computes h
// column 256*kb + t1_kmap(g, j), i.e. block kb of h in the down kernel's k order.  A 128-position
// work item is then the pair of k-groups {2p, 2p+1} of one block kb (p = (q >> 6) & 2), which is
// what one A scale of the down kernel's fp8 MFMA covers, so the item can scale each (row, block,
// pair) by itself.  Tiles of 16 positions are 16 consecutive columns, except that rows 12..15 of
// the tile at j = 48 are the group's four tail columns.  For I not a multiple of 256 (64, 128:
// no fp8 down kernel) the order is the identity.
__device__ __forceinline__ int t1_hcol(int q, int I) {
    if (I & 255) return q;
    return 256 * (q >> 8) + t1_kmap((q >> 6) & 3, q & 63);
}

template <int QT, int NMAT, int NTI, int MT, bool SPAN>
struct GuChunk {
    static constexpr int NT = NMAT * NTI;
    static constexpr int BB = Fmt<QT>::BYTES;
    static constexpr bool F16 = NMAT == 1;  // Q2B: down reads fp16 h, gate/up bf16 x
    typedef WinGeo<QT> G;

    const GuShared& sh;
    const BufSrc &srcx, &srcg, &srcu;
    const BufSrc &srcg_n, &srcu_n;  // weights of the next chunk
    const uint32_t* xoff;    // per lane: activation source offset of each of its GU_DMA loads
    const uint32_t* roff;    // per lane: byte offset of the row it decodes, per strip
    const uint32_t* woff;    // per lane: byte offset of its 16 bytes of a row window, per strip
    const uint32_t* woff_n;  // the same for the next chunk
    const uint32_t* wx;      // per strip: bytes added to quarter 3's offset beyond 12 rows (uniform)
    const uint32_t* wx_n;    // the same for the next chunk
    const uint32_t* xon;     // xoff of the next chunk (written by the hook)
    const T1Lane8& ln;
    int nkb, NS, wave, m, g;
    uint32_t rowb;           // bytes per weight row
    bool pf_next;            // load the next chunk's first windows and activation step
    bool pf_have;            // this chunk's were loaded by the chunk before
    typename StripDec<QT>::type dec[NT];
    RunScale rs[NT];
    f32x4 acc[MT][NT];

    typedef WinLay<QT, NT, NMAT, SPAN> WLay;
    __device__ __forceinline__ uint8_t* wbase() const { return sh.wts + wave * WLay::WAVE_BYTES; }
    // window of row r (0..15) of strip t
    __device__ __forceinline__ const uint32_t* win(int t, int r) const { return WLay::win(wbase(), t, r); }

    // step c of the activations into ring slot `slot`; c = NS: step 0 of the next chunk
    __device__ __forceinline__ void act(int c, int slot) {
        if (c < NS || pf_next) {
            uint8_t* base = sh.ring[slot] + wave * (GU_DMA * 1024);
            const uint32_t* xo = c < NS ? xoff : xon;
            const uint32_t so = c < NS ? act_step_off<QT>(c) : 0u;
#pragma unroll
            for (int i = 0; i < GU_DMA; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(srcx.r, (lds_void*)(base + i * 1024), 16, xo[i], so, 0, 0);
        }
    }
    // the windows of block kb (clamped to the last block, so that the number of loads is
    // fixed) of this wave's rows.  Narrow: in quarter q, lane L < 4*WL fetches its 16 bytes of the
    // window of row 4q + win_lane_row(L) (wo[t] holds lane L's offset for q = 0; rows are row_bytes
    // apart, except that quarter 3 of a strip may start wxx[t] bytes further on).  Wide: wo[q] is
    // lane L's offset in quarter q (see WinLay).
    __device__ __forceinline__ void wload_from(const BufSrc& sg, const BufSrc& su, const uint32_t* wo,
                                               const uint32_t* wxx, uint32_t blk) {
        if constexpr (WLay::ONE_RES) {  // (one resource: sg; for gate/up it spans both matrices)
#pragma unroll
            for (int i = 0; i < WLay::NOFF; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(sg.r, (lds_void*)(wbase() + WLay::load_lds_off(i)), 16,
                                                         (wo[i] + blk) & ~3u, 0, 0, 0);
        } else if ((threadIdx.x & 63) < 4 * G::WL) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        (t < NTI ? sg : su).r, (lds_void*)(wbase() + t * G::WS + G::WQ * q), 16,
                        (wo[t] + 4u * (uint32_t)q * rowb + (q == 3 ? wxx[t] : 0u) + blk) & ~3u, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void wload(int kb) {
        wload_from(srcg, srcu, woff, wx, (uint32_t)min(kb, nkb - 1) * BB);
    }
    // top of block kb: decoder state from this wave's windows, block scale into the
    // accumulators; then (its windows read) the next block's windows
    __device__ __forceinline__ void block_top(int kb) {
        // this block's windows were issued in the step before the last one; only that last
        // step's activation loads (GU_DMA) were issued after them
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(GU_DMA) : "memory");
        const uint32_t blk = (uint32_t)kb * BB;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            strip_prep<QT>(dec[t], win(t, m), (roff[t] + blk) & 3u, g, ln, sh);
            const float r = rs[t].step(dec[t].d);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt][t] *= r;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // windows read before they are replaced
    }
    // step c = 2*kb + H staged in ring slot H.  Even steps issue the next activation step and
    // then the next block's windows (so that no activation wait covers the windows, and they have
    // two steps to land); odd steps issue the next activation step only.
    template <int H, class Hook>
    __device__ __forceinline__ void step(int c, Hook& hook) {
        if (H == 0)
            vm_barrier<0>();
        else
            vm_barrier<WLay::LOADS>();
        // the hook's loads complete before the next step's wait
        if (c == NS - 2) hook();
        act(c + 1, 1 - H);
        if (H == 0) {
            const int kb = c >> 1;
            if (kb + 1 < nkb || !pf_next)
                wload(kb + 1);
            else
                wload_from(srcg_n, srcu_n, woff_n, wx_n, 0u);  // block 0 of the next chunk
        }
        mem_fence_compiler();
        int sa[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sa[mt] = 127;  // x rows: the per-row scale is applied after the K loop
        step_mfma<QT, F16, MT, NT, H>(dec, ln, sh, sh.ring[H], m, g, acc, sa);
        // the step's MFMAs are issued before the next step's barrier (not sunk past it, which
        // would keep two steps' operands live)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < NT; ++t) asm volatile("" : "+v"(acc[mt][t]));
    }

    template <class Hook>
    __device__ __forceinline__ void run(Hook& hook) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        // vector-memory operations complete in issue order, so the stores and loads before this
        // chunk only make the counted waits below stricter
        if (!pf_have) {
            act(0, 0);
            mem_fence_compiler();
            wload(0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // block 0's windows before they are read
        for (int kb = 0; kb < nkb; ++kb) {
            block_top(kb);
            step<0>(2 * kb, hook);
            step<1>(2 * kb + 1, hook);
        }
    }
};

// T1 gate/up output for the fp8 down kernel: h = silu(gate) * up of the chunk's rows goes straight
// into hi/lo fp8 rows in the down kernel's k order ([kb][h][g][hi 32 | lo 32], as the split of
// activation rows), scaled by 2^sigma per (row, work item) with max |h| * 2^sigma in [128, 256)
// over the item's 128 columns (block kb, k-groups 2p and 2p+1: one scale of the down MFMA);
// byte 2*kb + p of hsc[row] = 127 - sigma.  The maximum is a reduction over 16 lanes, then over
// the work-group's waves in LDS.
// maximum over the 16 lanes of a DPP row (row_ror 8, 4, 2, 1: no LDS round trips)
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));
    return x;
}

// ---------------------------------------------------------------------------------------
// Down epilogue: a wave's tile of per-pair outputs y into the slots (YSlots).
// yv[mt][t][i]: the wave's fp32 outputs, row r = 16*mt + 4*g + i of the chunk, column
// col0 + 16*t + n (t < 4: one 64-column tile); dst(r) = the row's pair index t*k + j, or >= P
// for a padding row, which is stored to the wave's own spare tile instead (never read; keeps
// padding stores of different waves off each other's cache lines).  A wave issues at least
// Y_STORE_OPS vector-memory stores per row tile (16 fp16 stores; the scaled case adds 4 sigma
// stores), which callers count in their waits.
constexpr int Y_STORE_OPS = 4 * 4;
template <int MT, class Dst>
__device__ __forceinline__ void y_store(const YSlots& c, float (&yv)[MT][4][4], Dst dst, int col0) {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    const int ntile = c.H / CT, tile = col0 / CT;
    const int wid = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));  // < Y_SPARE (host-checked)
    float lm = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t) lm = fmaxf(lm, fabsf(yv[mt][t][i]));
    if (__ballot(lm >= 32768.0f) == 0ull) {  // every value fits fp16 as it is (sigma = 0)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = dst(16 * mt + 4 * g + i);
                uint16_t* yr = d < c.P ? c.yslot + (size_t)d * c.H + col0 + n : c.yspare + (size_t)wid * CT + n;
#pragma unroll
                for (int t = 0; t < 4; ++t) yr[16 * t] = f32_to_f16_bits(yv[mt][t][i]);
            }
        return;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = fmaxf(fmaxf(fabsf(yv[mt][0][i]), fabsf(yv[mt][1][i])), fmaxf(fabsf(yv[mt][2][i]), fabsf(yv[mt][3][i])));
            m = row16_max(m);  // the 16 lanes of a DPP row hold the same rows
            const int ex = m > 0.f ? (int)((__float_as_uint(m) >> 23) & 255u) - 127 : 14;  // floor(log2 m)
            int sigma = 14 - ex;
            sigma = sigma < -120 ? -120 : (sigma > 120 ? 120 : sigma);
            const float sc = __uint_as_float((uint32_t)(127 + sigma) << 23);
            const int d = dst(16 * mt + 4 * g + i);
            const bool real = d < c.P;
            uint16_t* yr = real ? c.yslot + (size_t)d * c.H + col0 + n : c.yspare + (size_t)wid * CT + n;
            int8_t* ye = real ? c.yexp + (size_t)d * ntile + tile : c.espare + wid;
#pragma unroll
            for (int t = 0; t < 4; ++t) yr[16 * t] = f32_to_f16_bits(yv[mt][t][i] * sc);
            *ye = (int8_t)sigma;  // (the 16 lanes of a DPP row store the same byte)
        }
}

template <int MT, int NTI, class Ch>
__device__ __forceinline__ void t1_h_split_out(const GuArgs& a, const GuShared& sh, const Ch& ch, int pc, int rows,
                                               int colw, int wave, int n, int g) {
    // lane indices made opaque here, so that the compiler does not hoist the epilogue's
    // addresses out of the K loop (they would be spilled there)
    asm volatile("" : "+v"(n), "+v"(g));
    const int sb = colw >> 7;  // the item's scale byte, 2*kb + p
    float v[MT][4][NTI], pm[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float xs = sh.rscale[mt * 16 + 4 * g + i];  // 0 for rows past the chunk
            pm[mt][i] = 0.f;
#pragma unroll
            for (int ti = 0; ti < NTI; ++ti) {
                const float gv = ch.acc[mt][ti][i] * ch.rs[ti].dprev * xs;
                const float uv = ch.acc[mt][NTI + ti][i] * ch.rs[NTI + ti].dprev * xs;
                v[mt][i][ti] = silu_fast(gv) * uv;
                pm[mt][i] = fmaxf(pm[mt][i], fabsf(v[mt][i][ti]));
            }
        }
    // the 16 lanes n of lane group g hold the same rows
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) pm[mt][i] = row16_max(pm[mt][i]);
    if (n == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sh.hred[wave * 64 + mt * 16 + 4 * g + i] = pm[mt][i];
    }
    lds_barrier();
    float am[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = mt * 16 + 4 * g + i;
            am[mt][i] = fmaxf(fmaxf(sh.hred[r], sh.hred[64 + r]), fmaxf(sh.hred[128 + r], sh.hred[192 + r]));
        }
    static_assert(GU_NW == 4, "the work item's maximum spans the four waves");
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = mt * 16 + 4 * g + i;
            if (r < rows) {
                const float amax = am[mt][i];
                const int ex = amax > 0.f ? (int)((__float_as_uint(amax) >> 23) & 255u) - 127 : 7;
                int sigma = 7 - ex;
                sigma = sigma < -120 ? -120 : (sigma > 120 ? 120 : sigma);
                const float sc = __uint_as_float((uint32_t)(127 + sigma) << 23);
                uint8_t* drow = a.h8 + (size_t)(pc + r) * (size_t)(2 * a.N);
#pragma unroll
                for (int ti = 0; ti < NTI; ++ti) {
                    const int qc = colw + 16 * ti + n, j = qc & 63;
                    const int off = 512 * (qc >> 8) + 256 * (j >> 5) + 64 * ((qc >> 6) & 3) + (j & 31);
                    const float x = v[mt][i][ti] * sc;
                    const int hb = __builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false);
                    const int lb = __builtin_amdgcn_cvt_pk_fp8_f32(x - __builtin_amdgcn_cvt_f32_fp8(hb, 0), 0.f, 0, false);
                    drow[off] = (uint8_t)hb;
                    drow[off + 32] = (uint8_t)lb;
                }
                if (n == 0 && wave == 0) ((uint8_t*)a.hsc)[(size_t)(pc + r) * 4 + sb] = (uint8_t)(127 - sigma);
            }
        }
    // hred is rewritten only after the next chunk's step barriers
}

// One 64-pair chunk of a work item: K loop, then the epilogue (gate/up: SwiGLU into h; down:
// fp16 rows of y).  During the chunk's next-to-last step the hook gathers the next chunk's
// activation row offsets (xon), this chunk's per-row activation scales (ps; 1 for Q2B) and, for
// down, the rows' original pair indices (one row per thread of the first wave).
template <int QT, int MODE, int NTI, int MT, bool SPAN>
__device__ __forceinline__ void gu_chunk(const GuArgs& a, const GuShared& sh, const BufSrc& srcx,
                                         const BufSrc& srcg, const BufSrc& srcu, const BufSrc& srcg_n,
                                         const BufSrc& srcu_n, const uint32_t* xoff, const uint32_t* roff,
                                         const uint32_t* woff, const uint32_t* woff_n, const uint32_t* wx,
                                         const uint32_t* wx_n, const T1Lane8& ln, int nkb, int pc, int rows,
                                         int colw, bool has_next, bool pf_have, int pn, int rows_n, uint32_t* xon) {
    constexpr int NMAT = MODE == GU_GATEUP ? 2 : 1;
    const int tid = threadIdx.x, wave = uni(tid >> 6), lane = tid & 63, n = lane & 15, g = lane >> 4;
    float ps = 0.f;
    int pdst = a.P;  // padding rows: the spare tile
    auto hook = [&]() {
        if (has_next) {
#pragma unroll
            for (int i = 0; i < GU_DMA; ++i) {
                const int row = 4 * (wave * GU_DMA + i) + (lane >> 4);
                const int pr = pn + (row < rows_n ? row : 0);
                const int arow = MODE == GU_GATEUP ? a.pair_src[pr] / a.k : pr;
                xon[i] = (uint32_t)arow * (uint32_t)(2 * a.K) + act_piece_off<QT>((lane & 15) ^ (row & 15));
            }
        }
        if (tid < rows) {
            if constexpr (MODE == GU_GATEUP) {
                ps = QT == QT_T1 ? a.ascale[a.pair_src[pc + tid] / a.k] : 1.0f;
            } else {
                ps = QT == QT_T1 ? a.ascale[pc + tid] : 1.0f;
                pdst = a.pair_src[pc + tid];
            }
        }
    };
    GuChunk<QT, NMAT, NTI, MT, SPAN> ch{sh,   srcx,   srcg,   srcu, srcg_n, srcu_n, xoff, roff, woff,
                                  woff_n, wx,   wx_n,   xon,  ln,     nkb,    2 * nkb, wave, n,
                                  g,      (uint32_t)nkb * (uint32_t)Fmt<QT>::BYTES, has_next, pf_have};
    ch.run(hook);
    if (tid < 64) {
        sh.rscale[tid] = ps;
        if constexpr (MODE == GU_DOWN) sh.rdst[tid] = pdst;
    }
    lds_barrier();
    if constexpr (QT == QT_T1 && MODE == GU_GATEUP) {
        if (a.h8 != nullptr) {
            t1_h_split_out<MT, NTI>(a, sh, ch, pc, rows, colw, wave, n, g);
            return;
        }
    }
    if constexpr (MODE == GU_DOWN) {
        static_assert(MODE != GU_DOWN || NTI == 4, "a down wave covers one 64-column scale tile");
        float yv[MT][4][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float xs = sh.rscale[mt * 16 + 4 * g + i];  // 0 for padding rows
#pragma unroll
                for (int t = 0; t < 4; ++t) yv[mt][t][i] = ch.acc[mt][t][i] * ch.rs[t].dprev * xs;
            }
        y_store<MT>(a.ys, yv, [&](int r) { return sh.rdst[r]; }, colw);
    } else {
        // lane holds rows 4g..4g+3 of each 16-row tile, column n
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = mt * 16 + 4 * g + i;
                if (r < rows) {
                    const float xs = sh.rscale[r];
#pragma unroll
                    for (int ti = 0; ti < NTI; ++ti) {
                        const float gv = ch.acc[mt][ti][i] * ch.rs[ti].dprev * xs;
                        const float uv = ch.acc[mt][NTI + ti][i] * ch.rs[NTI + ti].dprev * xs;
                        const int hc = QT == QT_T1 ? t1_hcol(colw + 16 * ti + n, a.N) : colw + 16 * ti + n;
                        a.hbuf[(size_t)(pc + r) * a.N + hc] = f32_to_f16_bits(silu_fast(gv) * uv);
                    }
                }
            }
    }
    // rscale and rdst are rewritten only after the next chunk's step barriers
}

// Body of the gate/up kernels (and of the streamed down kernels for I > 512).
template <int QT, int MODE, int NTI, bool SPAN>
__device__ __forceinline__ void gu_kernel(const GuArgs& a) {
    constexpr int NTHR = 64 * GU_NW;
    constexpr int NT = (MODE == GU_GATEUP ? 2 : 1) * NTI;
    constexpr int BB = Fmt<QT>::BYTES;
    typedef GuTables<QT, MODE == GU_DOWN> Tab;
    // the decoder tables sit at the bottom of LDS (largest alignment first), so that their
    // constant offsets fit the 16-bit offset of LDS instructions
    __shared__ __attribute__((aligned(32768))) uint64_t t64[Tab::N64];
    __shared__ uint32_t tbl8[8];
    __shared__ float rscale[64];
    __shared__ int32_t rdst[64];
    typedef WinLay<QT, NT, MODE == GU_GATEUP ? 2 : 1, SPAN> WLay;
    __shared__ __attribute__((aligned(16))) uint8_t wts[GU_NW * WLay::WAVE_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t ring0[GU_STEP];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[GU_STEP];
    constexpr bool HCOL = QT == QT_T1 && MODE == GU_GATEUP;  // output columns in t1_hcol order
    __shared__ float hred[HCOL ? GU_NW * 64 : 1];
    const int tid = threadIdx.x, wave = uni(tid >> 6), lane = tid & 63, n = lane & 15, g = lane >> 4;
    const StaticSched sc(uni(*a.wl_len), a.ns, MODE == GU_GATEUP);
    if (sc.item(0) >= sc.nitems) return;  // uniform over the work-group
    Tab::build(t64, tbl8, tid, NTHR);
    GuShared sh0 = Tab::shared(ring0, ring1, wts, t64, tbl8, rscale, rdst);
    sh0.hred = hred;
    const GuShared sh = sh0;
    T1Lane8 ln;
    ln.init(g);
    const int nkb = a.K >> 8;
    const uint32_t row_bytes = (uint32_t)nkb * BB;
    const uint32_t mat_bytes = (uint32_t)a.N * row_bytes;
    const BufSrc srcx(a.act, 0x7FFFFFF0u);
    auto arow = [&](int p) { return MODE == GU_GATEUP ? a.pair_src[p] / a.k : p; };

    // first chunk: record and activation rows; later chunks are prefetched by their predecessor
    int q = 0, ix = sc.item(0), mc = 0;
    bool pf_have = false;  // the current chunk's first windows and activations were prefetched
    ItemRec rec = load_item(a.items, sc.rank(ix));
    uint32_t xoff[GU_DMA];
    {
        const int rows = min(64, rec.ne);
#pragma unroll
        for (int i = 0; i < GU_DMA; ++i) {
            const int row = 4 * (wave * GU_DMA + i) + (lane >> 4);
            const int ar = arow(rec.p0 + (row < rows ? row : 0));
            xoff[i] = (uint32_t)ar * (uint32_t)(2 * a.K) + act_piece_off<QT>((lane & 15) ^ (row & 15));
        }
    }
    __syncthreads();  // tables
    while (true) {
        // the chunk after this one (uniform)
        int qn = q, ixn = ix, mcn = mc + 64;
        ItemRec recn = rec;
        bool has_next = true;
        if (mcn >= rec.ne) {
            qn = q + 1;
            ixn = sc.item(qn);
            mcn = 0;
            has_next = ixn < sc.nitems;
            if (has_next) recn = load_item(a.items, sc.rank(ixn));
        }
        const int rows = min(64, rec.ne - mc);
        const int rows_n = has_next ? min(64, recn.ne - mcn) : 1;
        // wide gate/up windows: one resource from the lower of the gate and up matrices to the end
        // of the higher one, each lane's offsets relative to it
        constexpr bool COMB = WLay::ONE_RES && MODE == GU_GATEUP;
        const uint64_t lo = COMB ? min(rec.off[0], rec.off[1]) : rec.off[MODE == GU_GATEUP ? 0 : 2];
        const uint64_t lo_n = COMB ? min(recn.off[0], recn.off[1]) : recn.off[MODE == GU_GATEUP ? 0 : 2];
        const uint32_t span = COMB ? (uint32_t)(max(rec.off[0], rec.off[1]) - lo) + mat_bytes : mat_bytes;
        const uint32_t span_n = COMB ? (uint32_t)(max(recn.off[0], recn.off[1]) - lo_n) + mat_bytes : mat_bytes;
        const BufSrc srcg(a.arena + lo, span);
        const BufSrc srcu(a.arena + rec.off[1], mat_bytes);
        const BufSrc srcg_n(a.arena + lo_n, span_n);
        const BufSrc srcu_n(a.arena + recn.off[1], mat_bytes);
        const int colw = sc.slice(ix) * (16 * NTI * GU_NW) + wave * (16 * NTI);
        const int colw_n = sc.slice(ixn) * (16 * NTI * GU_NW) + wave * (16 * NTI);
        // weight row of output position c; quarter 3 of a strip starting at position c0 begins
        // at row col(c0 + 12), which for t1_hcol's tail tiles is not col(c0) + 12
        auto col = [&](int c) { return HCOL ? t1_hcol(c, a.N) : c; };
        uint32_t roff[NT], woff[WLay::NOFF], woff_n[WLay::NOFF], wx[NT], wx_n[NT];
        if constexpr (WLay::ONE_RES) {  // entry i: the lane's piece of load i (see WinLay)
#pragma unroll
            for (int i = 0; i < WLay::NOFF; ++i) {
                int tl, r, pc;
                WLay::lane_piece(i, lane, tl, r, pc);
                const int l0 = colw + 16 * (tl % NTI), l0n = colw_n + 16 * (tl % NTI);
                uint32_t mo = 0, mo_n = 0;  // the lane's matrix within the combined resource
                if constexpr (COMB) {
                    mo = (uint32_t)(rec.off[tl < NTI ? 0 : 1] - lo);
                    mo_n = (uint32_t)(recn.off[tl < NTI ? 0 : 1] - lo_n);
                }
                woff[i] = mo + (uint32_t)col(l0 + r) * row_bytes + 16u * (uint32_t)pc;
                woff_n[i] = mo_n + (uint32_t)col(l0n + r) * row_bytes + 16u * (uint32_t)pc;
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int c0 = colw + 16 * (t % NTI), c0n = colw_n + 16 * (t % NTI);
            roff[t] = (uint32_t)col(c0 + n) * row_bytes;
            if constexpr (WLay::ONE_RES) {
                wx[t] = wx_n[t] = 0u;
            } else {
                woff[t] = (uint32_t)col(c0 + win_lane_row<QT>(lane)) * row_bytes + win_lane_byte<QT>(lane);
                woff_n[t] = (uint32_t)col(c0n + win_lane_row<QT>(lane)) * row_bytes + win_lane_byte<QT>(lane);
                wx[t] = (uint32_t)(col(c0 + 12) - col(c0) - 12) * row_bytes;
                wx_n[t] = (uint32_t)(col(c0n + 12) - col(c0n) - 12) * row_bytes;
            }
        }
        uint32_t xon[GU_DMA];
#pragma unroll
        for (int i = 0; i < GU_DMA; ++i) xon[i] = xoff[i];
        const int pc = rec.p0 + mc, pn = recn.p0 + mcn;
#define RL_GU_CHUNK(MT_)                                                                                               \
    gu_chunk<QT, MODE, NTI, MT_, SPAN>(a, sh, srcx, srcg, srcu, srcg_n, srcu_n, xoff, roff, woff, woff_n, wx, wx_n, ln, nkb, \
                                 pc, rows, colw, has_next, pf_have, pn, rows_n, xon)
        switch ((rows + 15) >> 4) {
            case 1: RL_GU_CHUNK(1); break;
            case 2: RL_GU_CHUNK(2); break;
            case 3: RL_GU_CHUNK(3); break;
            default: RL_GU_CHUNK(4); break;
        }
#undef RL_GU_CHUNK
        if (!has_next) break;
        pf_have = true;
        q = qn;
        ix = ixn;
        mc = mcn;
        rec = recn;
#pragma unroll
        for (int i = 0; i < GU_DMA; ++i) xoff[i] = xon[i];
    }
}

// T1 experts on the fp8 MFMA: gate/up + SwiGLU (MODE GU_GATEUP), or down for I > 512 (GU_DOWN).
// SPAN: every expert's gate and up matrices lie within one buffer resource (the gate/up windows
// then take the wide layout, see WinLay); the host checks the descriptors.
template <int MODE, int NTI, bool SPAN>
__global__ __launch_bounds__(64 * GU_NW, 2) void k_t1_f8(GuArgs a) {
    gu_kernel<QT_T1, MODE, NTI, SPAN>(a);
}
// Q2B experts on the 16-bit MFMA: the same two uses
template <int MODE, int NTI, bool SPAN>
__global__ __launch_bounds__(64 * GU_NW, 2) void k_q2_mm(GuArgs a) {
    gu_kernel<QT_Q2B, MODE, NTI, SPAN>(a);
}

// ---------------------------------------------------------------------------------------
// Down with the activations held in LDS (K = I <= 512), both block types.  A work item is
// (expert, group of columns of H).  For each chunk of up to DN_ROWS of the expert's sorted pairs
// the work-group stages the chunk's activation rows once for all of K; then every wave sweeps its
// own columns, 16*DN_NT at a time, without work-group synchronisation: only its own weight
// windows move (the same windows, decoders and MFMA steps as the gate/up kernels).  y rows are
// fp16 at the pairs' original index; padding rows of a tile go to the spare row P of y.
constexpr int DN_ROWS = 48;
constexpr int DN_NT = 4;                     // strips of 16 columns per wave per sweep
constexpr int DN_SW = 16 * DN_NT * GU_NW;    // columns per sweep of the work-group
constexpr int DN_KMAX = 512;
constexpr int DN_ACT = DN_ROWS * 256;        // staged bytes per 128-value step

template <int QT, int MT>
struct DnSweep {
    static constexpr int NT = DN_NT;
    static constexpr int BB = Fmt<QT>::BYTES;
    typedef WinGeo<QT> G;

    const GuShared& sh;         // ring[0]: the chunk's activations [K/128 steps][DN_ROWS][256 B]
    const BufSrc &srcw, &srcw_n;  // down matrix of this sweep and of the next one
    const uint32_t* roff;       // per lane: byte offset of the row it decodes, per strip
    const uint32_t* woff;       // per lane: byte offset of its 16 bytes of a row window, per strip
    const uint32_t* woff_n;     // the same for the next sweep
    const T1Lane8& ln;
    int nkb, wave, m, g;
    uint32_t rowb;
    bool pf_next;               // load the next sweep's first windows during the last block
    bool pf_have;               // this sweep's first windows were loaded by the sweep before
    uint32_t rw[MT];            // T1: the scale word (hsc) of the lane's A row, per row tile
    int sa[MT];                 // T1: this block's A scale of the lane (127 = 1)
    typename StripDec<QT>::type dec[NT];
    RunScale rs[NT];
    f32x4 acc[MT][NT];

    typedef WinLay<QT, NT, 1> WLay;
    __device__ __forceinline__ uint8_t* wbase() const { return sh.wts + wave * WLay::WAVE_BYTES; }
    __device__ __forceinline__ const uint32_t* win(int t, int r) const { return WLay::win(wbase(), t, r); }
    // narrow: wo[t] is the lane's offset in quarter 0 of strip t; wide / linear: wo[i] its offset for load i
    __device__ __forceinline__ void wload_from(const BufSrc& sw, const uint32_t* wo, uint32_t blk) {
        if constexpr (WLay::ONE_RES) {
#pragma unroll
            for (int i = 0; i < WLay::NOFF; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(sw.r, (lds_void*)(wbase() + WLay::load_lds_off(i)), 16,
                                                         (wo[i] + blk) & ~3u, 0, 0, 0);
        } else if ((threadIdx.x & 63) < 4 * G::WL) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(sw.r, (lds_void*)(wbase() + t * G::WS + G::WQ * q), 16,
                                                             (wo[t] + 4u * (uint32_t)q * rowb + blk) & ~3u, 0, 0, 0);
        }
    }
    // windows of block kb: the wave's own loads, so a wait on its own counter suffices.  At the
    // first block of a sweep the previous sweep's epilogue (y_store) has issued exactly
    // Y_STORE_OPS * MT stores after this sweep's windows: waiting down to that many outstanding
    // operations completes the windows without waiting for those stores.  (The first sweep of a
    // chunk follows a full wait.)
    __device__ __forceinline__ void block_top(int kb) {
        if (kb == 0)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Y_STORE_OPS * MT) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const uint32_t blk = (uint32_t)kb * BB;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            strip_prep<QT>(dec[t], win(t, m), (roff[t] + blk) & 3u, g, ln, sh);
            const float r = rs[t].step(dec[t].d);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt][t] *= r;
        }
        // lane group g supplies the scale of k-group pair g & 1 (see mfma_f8)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            sa[mt] = QT == QT_T1 ? (int)((rw[mt] >> (16 * kb + 8 * (g & 1))) & 255u) : 127;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // windows read before they are replaced
        if (kb + 1 < nkb)
            wload_from(srcw, woff, (uint32_t)(kb + 1) * BB);
        else if (pf_next)
            wload_from(srcw_n, woff_n, 0u);
    }
    template <int H>
    __device__ __forceinline__ void step(int c) {
        step_mfma<QT, true, MT, NT, H>(dec, ln, sh, sh.ring[0] + c * DN_ACT, m, g, acc, sa);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < NT; ++t) asm volatile("" : "+v"(acc[mt][t]));
    }
    __device__ __forceinline__ void run() {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!pf_have) wload_from(srcw, woff, 0u);
        for (int kb = 0; kb < nkb; ++kb) {
            block_top(kb);
            step<0>(2 * kb);
            step<1>(2 * kb + 1);
        }
    }
};

// All sweeps of one chunk (MT row tiles) of a work item: columns cbase + s*DN_SW, s < nsw.
template <int QT, int MT>
__device__ __forceinline__ void dn_chunk(const GuArgs& a, const GuShared& sh, const BufSrc& srcw,
                                         const BufSrc& srcw_next_item, const T1Lane8& ln, int nkb, uint32_t rowb,
                                         int cbase, int nsw, int cbase_next, bool next_item, const uint32_t* rsc) {
    const int tid = threadIdx.x, wave = uni(tid >> 6), lane = tid & 63, n = lane & 15, g = lane >> 4;
    bool pf_have = true;  // the first sweep's windows were loaded before the chunk's staging
    // scale word of the lane's A row (row mt*16 + n) in each row tile
    uint32_t rw[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) rw[mt] = rsc[mt * 16 + n];
    for (int s = 0; s < nsw; ++s) {
        const int col0 = cbase + s * DN_SW + wave * (16 * DN_NT);
        const bool last = s + 1 == nsw;
        const int col0n = last ? cbase_next + wave * (16 * DN_NT) : col0 + DN_SW;
        typedef WinLay<QT, DN_NT, 1> WLay;
        uint32_t roff[DN_NT], woff[WLay::NOFF], woff_n[WLay::NOFF];
        if constexpr (WLay::ONE_RES) {  // entry i: the lane's piece of load i
#pragma unroll
            for (int i = 0; i < WLay::NOFF; ++i) {
                int tl, r, pc;
                WLay::lane_piece(i, lane, tl, r, pc);
                woff[i] = ((uint32_t)col0 + (uint32_t)(16 * tl + r)) * rowb + 16u * (uint32_t)pc;
                woff_n[i] = ((uint32_t)col0n + (uint32_t)(16 * tl + r)) * rowb + 16u * (uint32_t)pc;
            }
        }
#pragma unroll
        for (int t = 0; t < DN_NT; ++t) {
            roff[t] = (uint32_t)(col0 + 16 * t + n) * rowb;
            if constexpr (WLay::ONE_RES) {
            } else {
                woff[t] = ((uint32_t)(col0 + 16 * t) + win_lane_row<QT>(lane)) * rowb + win_lane_byte<QT>(lane);
                woff_n[t] = ((uint32_t)(col0n + 16 * t) + win_lane_row<QT>(lane)) * rowb + win_lane_byte<QT>(lane);
            }
        }
        DnSweep<QT, MT> sw{sh,  srcw, last ? srcw_next_item : srcw, roff, woff, woff_n, ln, nkb, wave, n, g, rowb,
                           !last || next_item, pf_have};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sw.rw[mt] = rw[mt];
        sw.run();
        // y tile of the wave (padding rows: rdst = P)
        static_assert(DN_NT == 4, "a down wave covers one 64-column scale tile");
        float yv[MT][4][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int t = 0; t < DN_NT; ++t) yv[mt][t][i] = sw.acc[mt][t][i] * sw.rs[t].dprev;
        y_store<MT>(a.ys, yv, [&](int r) { return sh.rdst[r]; }, col0);
        pf_have = true;
    }
}

template <int QT>
__device__ __forceinline__ void dn_kernel(const GuArgs& a) {
    constexpr int NTHR = 64 * GU_NW;
    constexpr int BB = Fmt<QT>::BYTES;
    typedef WinGeo<QT> G;
    typedef GuTables<QT, true> Tab;
    __shared__ __attribute__((aligned(32768))) uint64_t t64[Tab::N64];
    __shared__ uint32_t tbl8[8];
    __shared__ uint32_t rsc[DN_ROWS];  // T1: the rows' scale words (hsc)
    __shared__ int32_t rdst[DN_ROWS];
    typedef WinLay<QT, DN_NT, 1> WLay;
    __shared__ __attribute__((aligned(16))) uint8_t wts[GU_NW * WLay::WAVE_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t actb[(DN_KMAX / 128) * DN_ACT];
    const int tid = threadIdx.x, wave = uni(tid >> 6), lane = tid & 63, g = lane >> 4;
    const StaticSched sc(uni(*a.wl_len), a.ns);
    if (sc.item(0) >= sc.nitems) return;  // uniform over the work-group
    Tab::build(t64, tbl8, tid, NTHR);
    const GuShared sh = Tab::shared(actb, actb, wts, t64, tbl8, nullptr, rdst);
    T1Lane8 ln;
    ln.init(g);
    const int nkb = a.K >> 8, NS = 2 * nkb;
    const uint32_t rowb = (uint32_t)nkb * BB;
    const uint32_t mat_bytes = (uint32_t)a.N * rowb;
    const int P = a.P;  // y row P is the spare row
    const BufSrc srcx(a.act, 0x7FFFFFF0u);
    const int cw = a.N / a.ns;        // columns per item
    const int nsw = cw / DN_SW;
    // staging of a chunk: 12*NS loads of 1 KB (each 4 rows x 256 bytes of one step), shared by
    // the waves (12*NS is a multiple of 24, so of GU_NW)
    static_assert(24 % GU_NW == 0, "staging loads split evenly over the waves");
    const int npw = 12 * NS / GU_NW;
    auto stage = [&](int pc, int rows) {
#pragma unroll 4
        for (int j = 0; j < npw; ++j) {
            const int J = wave * npw + j;            // 0 .. 12*NS-1
            const int c = J / 12, rg = J % 12;
            const int row = 4 * rg + (lane >> 4);
            const int pr = pc + (row < rows ? row : 0);
            const uint32_t off = (uint32_t)pr * (uint32_t)(2 * a.K) + act_step_off<QT>(c) +
                                 act_piece_off<QT>((lane & 15) ^ (row & 15));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(srcx.r, (lds_void*)(actb + c * DN_ACT + rg * 1024), 16, off, 0, 0, 0);
        }
        if (tid < DN_ROWS) {
            rsc[tid] = QT == QT_T1 && tid < rows ? a.hsc[pc + tid] : 0x7F7F7F7Fu;
            rdst[tid] = tid < rows ? a.pair_src[pc + tid] : P;
        }
    };
    int q = 0, ix = sc.item(0), mc = 0;
    ItemRec rec = load_item(a.items, sc.rank(ix));
    __syncthreads();  // tables
    bool first = true;
    while (true) {
        int qn = q, ixn = ix, mcn = mc + DN_ROWS;
        ItemRec recn = rec;
        bool has_next = true;
        if (mcn >= rec.ne) {
            qn = q + 1;
            ixn = sc.item(qn);
            mcn = 0;
            has_next = ixn < sc.nitems;
            if (has_next) recn = load_item(a.items, sc.rank(ixn));
        }
        const int rows = min(DN_ROWS, rec.ne - mc);
        const BufSrc srcw(a.arena + rec.off[2], mat_bytes);
        const BufSrc srcw_n(a.arena + recn.off[2], mat_bytes);
        const int cbase = sc.slice(ix) * cw, cbase_n = sc.slice(ixn) * cw;
        if (!first) __syncthreads();  // every wave is done with the previous chunk's activations
        stage(rec.p0 + mc, rows);
        if (first) {  // the first sweep's windows (later ones are loaded by the sweep before)
            const int col0 = cbase + wave * (16 * DN_NT);
            uint8_t* wb = wts + wave * WLay::WAVE_BYTES;
            if constexpr (WLay::ONE_RES) {
#pragma unroll
                for (int i = 0; i < WLay::NOFF; ++i) {
                    int tl, r, pc;
                    WLay::lane_piece(i, lane, tl, r, pc);
                    const uint32_t wo = ((uint32_t)col0 + (uint32_t)(16 * tl + r)) * rowb + 16u * (uint32_t)pc;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(srcw.r, (lds_void*)(wb + WLay::load_lds_off(i)), 16, wo & ~3u,
                                                             0, 0, 0);
                }
            } else if ((lane & 63) < 4 * G::WL) {
#pragma unroll
                for (int t = 0; t < DN_NT; ++t)
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const uint32_t wo = ((uint32_t)(col0 + 16 * t) + win_lane_row<QT>(lane)) * rowb +
                                            win_lane_byte<QT>(lane);
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(srcw.r, (lds_void*)(wb + t * G::WS + G::WQ * qq),
                                                                 16, (wo + 4u * (uint32_t)qq * rowb) & ~3u, 0, 0, 0);
                    }
            }
            first = false;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // the chunk's activations and row tables
        switch ((rows + 15) >> 4) {
            case 1: dn_chunk<QT, 1>(a, sh, srcw, srcw_n, ln, nkb, rowb, cbase, nsw, cbase_n, has_next, rsc); break;
            case 2: dn_chunk<QT, 2>(a, sh, srcw, srcw_n, ln, nkb, rowb, cbase, nsw, cbase_n, has_next, rsc); break;
            default: dn_chunk<QT, 3>(a, sh, srcw, srcw_n, ln, nkb, rowb, cbase, nsw, cbase_n, has_next, rsc); break;
        }
        if (!has_next) break;
        q = qn;
        ix = ixn;
        mc = mcn;
        rec = recn;
    }
}

// T1 down on the fp8 MFMA, and Q2B down on the fp16 MFMA, for I <= 512
__global__ __launch_bounds__(64 * GU_NW, 2) void k_t1_dn(GuArgs a) { dn_kernel<QT_T1>(a); }
__global__ __launch_bounds__(64 * GU_NW, 2) void k_q2_dn(GuArgs a) { dn_kernel<QT_Q2B>(a); }

struct DownArgs {
    const uint16_t* hbuf;  // [P][I] fp16, sorted-pair order
    const uint8_t* arena;
    const int32_t* pair_src;
    const ItemRec* items;  // this type's work records
    const int32_t* wl_len;
    int32_t* counters;
    YSlots ys;        // the per-pair outputs
    int32_t* flags;
    int H, I, ns;
};

template <int QT, int LCH, int NW, int NTW, int MT>
__device__ __forceinline__ void down_chunk(const DownArgs& a, const DecodeTables<QT, true>& tab,
                                           uint16_t (*As)[64 * ChunkShape<(LCH / 32 < 4 ? LCH / 32 : 4), 64 * NW>::LDA],
                                           const BufSrc& srch, const BufSrc& src,
                                           Stager<(LCH / 32 < 4 ? LCH / 32 : 4), 64 * NW>& sx, int col0,
                                           f32x4 (&acc)[4][NTW], RunScale* rs) {
    constexpr int BB = Fmt<QT>::BYTES;
    constexpr int STRIP = LCH / 4;
    constexpr int NFRAG = STRIP / 8;
    constexpr int CS = NFRAG < 4 ? NFRAG : 4;  // steps per chunk
    constexpr int CPB = NFRAG / CS;            // chunks per K block
    using CH = ChunkShape<CS, 64 * NW>;
    const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
    const int nkc = a.I / LCH;
    StripRaw<QT, STRIP> raw[NTW];
    Strip<QT, STRIP> st[NTW];
    auto rload = [&](int kc) {
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
            const uint32_t flat = (uint32_t)(col0 + 16 * t + n) * (uint32_t)a.I + (uint32_t)kc * LCH;
            raw[t].load(src, (flat >> 8) * BB, (int)(flat & 255) + STRIP * g);
        }
    };
    auto koff = [&](int c) { return 2u * (uint32_t)((c / CPB) * LCH + (c % CPB) * CH::SEG); };
    const int nch = CPB * nkc;
    rload(0);
    sx.load(srch, 0u, tid);
    __syncthreads();
    sx.store(As[0], tid);
    if (nch > 1) sx.load(srch, koff(1), tid);
    __syncthreads();
    for (int kc = 0; kc < nkc; ++kc) {
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
            st[t].prepare(raw[t], tab.tern);
            const float r = rs[t].step(st[t].d);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt][t] *= r;
            __builtin_amdgcn_sched_barrier(0);  // one tile's table lookups in flight at a time
        }
        if (kc + 1 < nkc) rload(kc + 1);
#pragma unroll
        for (int part = 0; part < CPB; ++part) {
            const int c = CPB * kc + part;
            const uint16_t* Ab = As[c & 1];
#pragma unroll
            for (int f4 = 0; f4 < CS; ++f4) {
                u32x4 b[NTW];
#pragma unroll
                for (int t = 0; t < NTW; ++t) b[t] = st[t].frag(CS * part + f4, tab.val);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const u32x4 av = *(const u32x4*)&Ab[(mt * 16 + n) * CH::LDA + CH::SEG * g + 8 * f4];
#pragma unroll
                    for (int t = 0; t < NTW; ++t) acc[mt][t] = mfma_f16(av, b[t], acc[mt][t]);
                }
                __builtin_amdgcn_sched_barrier(0);  // bound the operands in flight to one step
            }
            if (c + 1 < nch) sx.store(As[(c + 1) & 1], tid);
            if (c + 2 < nch) sx.load(srch, koff(c + 2), tid);
            __syncthreads();
        }
    }
}

// One work item = one expert x (16*NTW*NW) output columns.  K runs over the intermediate
// dimension in blocks of LCH = min(I, 256) values (each inside one block of every W_down row);
// lane (n, g) decodes values LCH/4*g .. LCH/4*(g+1)-1 of each; activation chunks as k_gateup.
template <int QT, int LCH, int NW, int NTW>
__global__ __launch_bounds__(64 * NW, 512 / (64 * NW)) void k_down(DownArgs a) {
    constexpr int NTHR = 64 * NW;
    constexpr int BB = Fmt<QT>::BYTES;
    constexpr int STRIP = LCH / 4;
    constexpr int NFRAG = STRIP / 8;
    constexpr int CS = NFRAG < 4 ? NFRAG : 4;
    using CH = ChunkShape<CS, NTHR>;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][64 * CH::LDA];
    __shared__ DecodeTables<QT, true> tab;
    __shared__ int item_sh;
    const int tid = threadIdx.x, wave = tid >> 6;
    tab.build(tid, NTHR);
    __syncthreads();
    const int n_ranks = uni(*a.wl_len);
    const uint32_t mat_bytes = (uint32_t)((size_t)a.H * a.I / 256 * BB);
    const BufSrc srch(a.hbuf, 0x7FFFFFF0u);
    int rank, slice;
    while (next_item(a.counters, a.ns, n_ranks, &item_sh, rank, slice)) {
        const ItemRec rec = load_item(a.items, rank);
        const int p0 = rec.p0, ne = rec.ne;
        const BufSrc src(a.arena + rec.off[2], mat_bytes);
        const int col0 = slice * (16 * NTW * NW) + wave * (16 * NTW);

        for (int mc = 0; mc < ne; mc += 64) {
            const int rows = min(64, ne - mc);
            const int mtiles = (rows + 15) >> 4;
            Stager<CS, NTHR> sx;
#pragma unroll
            for (int i = 0; i < CH::PER_THREAD; ++i) {
                const int idx = tid + NTHR * i;
                const int row = idx / CH::PIECES, pc = idx % CH::PIECES;
                sx.off[i] = 2u * ((uint32_t)(p0 + mc + (row < rows ? row : 0)) * (uint32_t)a.I +
                                  (uint32_t)(STRIP * (pc / (CH::PIECES / 4)) + 8 * (pc % (CH::PIECES / 4))));
            }
            f32x4 acc[4][NTW];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int t = 0; t < NTW; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            RunScale rs[NTW];
            switch (mtiles) {
                case 1: down_chunk<QT, LCH, NW, NTW, 1>(a, tab, As, srch, src, sx, col0, acc, rs); break;
                case 2: down_chunk<QT, LCH, NW, NTW, 2>(a, tab, As, srch, src, sx, col0, acc, rs); break;
                case 3: down_chunk<QT, LCH, NW, NTW, 3>(a, tab, As, srch, src, sx, col0, acc, rs); break;
                default: down_chunk<QT, LCH, NW, NTW, 4>(a, tab, As, srch, src, sx, col0, acc, rs); break;
            }
            // y tile of the wave
            static_assert(NTW == 4, "a down wave covers one 64-column scale tile");
            const int32_t* psrc = a.pair_src + p0 + mc;
            auto dst = [&](int r) { return r < rows ? psrc[r] : a.ys.P; };
#define RL_KD_EPI(MT_)                                                                  \
    {                                                                                   \
        float yv[MT_][4][4];                                                            \
        for (int mt = 0; mt < MT_; ++mt)                                                \
            for (int i = 0; i < 4; ++i)                                                 \
                for (int t = 0; t < 4; ++t) yv[mt][t][i] = acc[mt][t][i] * rs[t].dprev; \
        y_store<MT_>(a.ys, yv, dst, col0);                                              \
    }
            switch (mtiles) {
                case 1: RL_KD_EPI(1); break;
                case 2: RL_KD_EPI(2); break;
                case 3: RL_KD_EPI(3); break;
                default: RL_KD_EPI(4); break;
            }
#undef RL_KD_EPI
        }
    }
}

// Weights of the ordered combine: selection j < kin of token t weighs w[t*kin + j]; with a shared
// expert (gate != NULL) the last selection (j = kin) weighs gate[t]; res (may be NULL) is added
// after the whole sum.
struct CombineW {
    const float* w;     // [T][kin]
    const float* gate;  // [T] or NULL
    const float* res;   // [T][H] or NULL
    int kin;
};

// The ordered weighted combine (the MoE tail): out[t][c] = sum over j = 0..K-1, in selection
// order, of weight(t, j) * y_{t,j}[c] (then + res[t][c]), with y read from the slots (fp16 *
// 2^-sigma per 64-column tile, exact in fp32).  One work-group per token, eight columns per thread
// (16-byte loads), one instance per K (1..16 pairs per token).  A separate pass: the K outputs of
// a token come from K experts on different XCDs, and making them visible to a last-arriving wave
// inside the down kernels costs more than this pass (L2 writebacks or device-coherent stores per
// tile).
template <int K>
__global__ __launch_bounds__(256) void k_combine(YSlots ys, CombineW cw, float* __restrict__ out) {
    const int t = blockIdx.x, H = ys.H, ntile = H / CT;
    float wt[K];
#pragma unroll
    for (int j = 0; j < K; ++j)
        wt[j] = (cw.gate != nullptr && j == K - 1) ? cw.gate[t] : cw.w[(size_t)t * cw.kin + j];
    for (int c = 8 * threadIdx.x; c < H; c += 8 * 256) {
        // the K rows' loads are all in flight before the first product
        u32x4 y[K];
        int e[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            y[j] = *(const u32x4*)(ys.yslot + ((size_t)t * K + j) * H + c);
            e[j] = ys.yexp[((size_t)t * K + j) * ntile + c / CT];
        }
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const float s = __uint_as_float((uint32_t)(127 - e[j]) << 23);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = __fmaf_rn(wt[j], half_bits_to_float(y[j][i] & 0xFFFFu) * s, acc[2 * i]);
                acc[2 * i + 1] = __fmaf_rn(wt[j], half_bits_to_float(y[j][i] >> 16) * s, acc[2 * i + 1]);
            }
        }
        if (cw.res != nullptr) {
            const f32x4* r = (const f32x4*)(cw.res + (size_t)t * H + c);
            const f32x4 r0 = r[0], r1 = r[1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i] += r0[i];
                acc[4 + i] += r1[i];
            }
        }
        f32x4* o = (f32x4*)(out + (size_t)t * H + c);
        o[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
        o[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
}

// ---------------------------------------------------------------------------------------
// 1-2 row path (decode and 2-row verify).  Memory-bound: every weight is read once per row.
// Types present are a template mask (1: Q2B, 2: T1, 3: both; both tables are then in LDS).
// Weights are decoded to exact 16-bit operands (bf16 against x, fp16 against h) and multiplied
// two at a time by the packed dot products v_dot2_f32_bf16 / v_dot2_f32_f16 (fp32 sums).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Decode tables of the 1-2 row kernels: the unit row (s = 1) of the value table, i.e. the
// operands (c - 1) (T1) or (2c - 3) (Q2B) of every byte of four codes, and the T1 digit table;
// the sub-scale multiplies each sub-scale group's partial sum instead (2 KB of values instead of
// 16 KB for T1 and 32 KB for Q2B, so a work-group's copy is short).
template <int QT, bool F16>
struct alignas(16) GvUnitTables {
    uint64_t val[256];
    uint32_t tern[QT == QT_T1 ? 256 : 4];  // (Q2B: padding to whole 16-byte units)
};
template <int QT, bool F16>
constexpr GvUnitTables<QT, F16> make_unit_tables() {
    GvUnitTables<QT, F16> t{};
    for (int i = 0; i < 256; ++i) t.val[i] = val_entry<QT, F16>(256 + i);
    if constexpr (QT == QT_T1)
        for (int i = 0; i < 256; ++i) t.tern[i] = tern_entry((uint32_t)i);
    return t;
}
template <int QT, bool F16>
__device__ constexpr GvUnitTables<QT, F16> kGvUnitTables = make_unit_tables<QT, F16>();
template <int QT, bool F16>
__device__ __forceinline__ void copy_unit_tables(GvUnitTables<QT, F16>& dst, int tid, int nthr) {
    static_assert(sizeof(GvUnitTables<QT, F16>) % 16 == 0, "whole 16-byte units");
    constexpr int N = (int)(sizeof(GvUnitTables<QT, F16>) / 16);
    const u32x4* s = reinterpret_cast<const u32x4*>(&kGvUnitTables<QT, F16>);
    u32x4* d = reinterpret_cast<u32x4*>(&dst);
    for (int i = tid; i < N; i += nthr) d[i] = s[i];
}

// The decoder of the 1-2 row kernels, run as they run it: the unit-row tables copied from the
// initialised device data, a strip's raw bytes through the buffer loads of StripRaw, the unit
// operands of frag1 (bf16 for gate/up, F16 = false; fp16 for down, F16 = true), then the strip's
// sub-scale and the block scale.  Block b is cut into strips of 64, 32 or 16 values by b % 3, so
// that one call covers the three strip widths; thread j of a block's 16 decodes its strip j (when
// the block has that many).  (unit * sub) * d is exact in fp32.
template <int QT, int S, bool F16>
__device__ __forceinline__ void dequant_rows_strip(const BufSrc& src, uint32_t mis, int j,
                                                   const GvUnitTables<QT, F16>& tb, float* o) {
    typedef Strip<QT, S> St;
    StripRaw<QT, S> raw;
    raw.load(src, mis, S * j);
    St st;
    st.prepare(raw, tb.tern);
#pragma unroll
    for (int f = 0; f < S / 8; ++f) {
        const u32x4 fr = st.frag1(f, tb.val);
        const float sc = st.sub(f / St::FPS);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = fr[i];
            float u0, u1;
            if constexpr (F16) {
                u0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
                u1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
            } else {
                u0 = __uint_as_float(w << 16);
                u1 = __uint_as_float(w & 0xFFFF0000u);
            }
            o[S * j + 8 * f + 2 * i] = (u0 * sc) * st.d;
            o[S * j + 8 * f + 2 * i + 1] = (u1 * sc) * st.d;
        }
    }
}

template <int QT, bool F16>
__global__ __launch_bounds__(256) void k_dequant_rows(const uint8_t* __restrict__ blocks, int64_t n_blocks,
                                                      float* __restrict__ out) {
    __shared__ GvUnitTables<QT, F16> tb;
    copy_unit_tables(tb, threadIdx.x, 256);
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n_blocks * 16) return;
    const int64_t b = t >> 4;
    const int j = (int)(t & 15);
    const uintptr_t base = (uintptr_t)(blocks + b * Fmt<QT>::BYTES);
    const uint32_t mis = (uint32_t)(base & 3);
    const BufSrc src((const uint8_t*)(base - mis), mis + Fmt<QT>::BYTES);
    float* o = out + b * 256;
    switch ((int)(b % 3)) {
        case 0:
            if (j < 4) dequant_rows_strip<QT, 64, F16>(src, mis, j, tb, o);
            break;
        case 1:
            if (j < 8) dequant_rows_strip<QT, 32, F16>(src, mis, j, tb, o);
            break;
        default:
            dequant_rows_strip<QT, 16, F16>(src, mis, j, tb, o);
            break;
    }
}

struct NoTables {};
// only the tables of the types present take LDS (T1 alone: 3 KB, Q2B alone: 2 KB)
template <int QMASK, bool F16>
struct GvTables {
    std::conditional_t<(QMASK & 1) != 0, GvUnitTables<QT_Q2B, F16>, NoTables> q2b;
    std::conditional_t<(QMASK & 2) != 0, GvUnitTables<QT_T1, F16>, NoTables> t1;
    __device__ inline void load(int tid, int nthr) {
        if constexpr (QMASK & 1) copy_unit_tables(q2b, tid, nthr);
        if constexpr (QMASK & 2) copy_unit_tables(t1, tid, nthr);
    }
};

// sum over the S values of one strip (inside one block) of w_i * xs[i], times the block scale;
// xs is bf16 bits (XS_BF16, weights decoded to bf16) or fp16 bits (weights decoded to fp16).
// Fixed order: per sub-scale group, pairs (2i, 2i+1) ascending of the unit operands, times the
// sub-scale, groups ascending, then the block scale.
template <int QT, int S, bool XS_BF16>
__device__ __forceinline__ float strip_dot_raw(const StripRaw<QT, S>& raw, const uint16_t* xs,
                                               const GvUnitTables<QT, !XS_BF16>& tb) {
    typedef Strip<QT, S> St;
    St st;
    st.prepare(raw, tb.tern);
    float part = 0.f;
#pragma unroll
    for (int gi = 0; gi < St::NSB; ++gi) {
        float pg = 0.f;
#pragma unroll
        for (int f = gi * St::FPS; f < (gi + 1) * St::FPS && f < S / 8; ++f) {
            const u32x4 fr = st.frag1(f, tb.val);
            const u32x4 xv = *(const u32x4*)(xs + 8 * f);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // through scalars: a bit_cast straight from a vector element reads element 0 only
                // with this compiler
                const uint32_t fw = fr[i], xw = xv[i];
                if constexpr (XS_BF16)
                    pg = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, fw), __builtin_bit_cast(bf16x2, xw), pg,
                                                         false);
                else
                    pg = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, fw), __builtin_bit_cast(f16x2, xw), pg, false);
            }
        }
        part = __fmaf_rn(st.sub(gi), pg, part);
    }
    return part * st.d;
}

// nst (<= MAXS) strips of S values of row `row` of a [rows x C] matrix, starting at column c0:
// the sum over the strips in ascending order.  All the strips' loads are issued before the first
// is decoded, so a lane waits for memory once.
template <int QT, int S, int MAXS, bool XS_BF16>
__device__ __forceinline__ float row_dot_t(const BufSrc& src, int C, int row, int c0, int nst, const uint16_t* xs,
                                           const GvUnitTables<QT, !XS_BF16>& tb) {
    StripRaw<QT, S> raw[MAXS];
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
        if (s < nst) {
            const uint32_t flat = (uint32_t)row * (uint32_t)C + (uint32_t)(c0 + s * S);
            raw[s].load(src, (flat >> 8) * Fmt<QT>::BYTES, (int)(flat & 255));
        }
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
        if (s < nst)
            acc += strip_dot_raw<QT, S, XS_BF16>(raw[s], xs + s * S, tb);
    return acc;
}

template <int QMASK, int S, int MAXS, bool XS_BF16>
__device__ __forceinline__ float row_dot(int qtype, const uint8_t* W, uint32_t mat_bytes, int C, int row, int c0,
                                         int span, const uint16_t* xs, const GvTables<QMASK, !XS_BF16>& tb) {
    const BufSrc src(W, mat_bytes);
    const int nst = span / S;
    if constexpr (QMASK & 2) {
        if (QMASK == 2 || qtype == QT_T1) return row_dot_t<QT_T1, S, MAXS, XS_BF16>(src, C, row, c0, nst, xs, tb.t1);
    }
    if constexpr (QMASK & 1) return row_dot_t<QT_Q2B, S, MAXS, XS_BF16>(src, C, row, c0, nst, xs, tb.q2b);
    return 0.f;
}

// The call's pairs (R*k <= 32): expert (-1 for an id outside [0, E)), type and matrix offsets.
// The gate/up kernel resolves them (ids, then descriptors) into LDS, so that a wave's weight
// loads wait on LDS, and its first work-group stores the table for the down kernel, which then
// reads it with one load instead of two dependent ones.
struct GvPair {
    int32_t e, qt;
    uint64_t gate_off, up_off, down_off;
};
constexpr int GV_MAX_PAIRS = 32;

struct GvArgs {
    const uint16_t* x;
    PairIds pid;      // the call's pairs (k = pid.kk per row, the last one the shared expert if any)
    const float* w;   // [R][pid.kin]
    const float* gate;  // [R]: weight of the shared expert's pair (with pid.shared >= 0)
    const float* res;   // [R][H] or NULL: added after the ordered sum
    const uint8_t* arena;
    const rl_expert_desc* desc;
    uint16_t* hgv;  // [R*k][I] fp16
    GvPair* pairs;  // [R*k]: written by the gate/up kernel, read by the down kernel
    float* out;  // [R][H]
    int32_t* flags;
    int R, k, E, H, I;
    __device__ __forceinline__ float weight(int p) const {  // weight of pair p = r*k + j
        if (pid.shared < 0) return w[p];
        const int r = p / k, j = p - r * k;
        return j < pid.kin ? w[r * pid.kin + j] : gate[r];
    }
};


__device__ __forceinline__ void gv_load_pairs(const GvArgs& a, GvPair* sp) {
    const int tid = threadIdx.x;
    if (tid < a.R * a.k) {
        const int e = a.pid.expert(tid);
        GvPair p{-1, 0, 0, 0, 0};
        if (e >= 0 && e < a.E) {
            const rl_expert_desc d = a.desc[e];
            p = GvPair{e, d.qtype, d.gate_off, d.up_off, d.down_off};
        }
        sp[tid] = p;
    }
}

// A wave computes features i0, i0+1 of one (row, slot) pair: lanes 0-15 gate row i0, 16-31
// gate i0+1, 32-47 up i0, 48-63 up i0+1; each lane covers H/16 consecutive values (two lanes
// per 256-value block when H = 2048), then a fixed xor tree reduces the 16 partial sums.
// x (R rows, 16-byte aligned) is staged in LDS once per work-group: each lane reads H/16 values
// of it per row, which through the vector memory path cost more than the weight loads.  Every
// run of H/16 values (one lane's share) is followed by 16 bytes of padding, so that the 16 lanes
// of a row, reading at the same offset of their runs, fall on different LDS banks.  Dynamic LDS
// of gv_xs_bytes(R, H) bytes.
__host__ __device__ constexpr int gv_xs_row(int H) { return H + 16 * 8; }  // halfwords per staged row
__host__ __device__ constexpr size_t gv_xs_bytes(int R, int H) { return (size_t)R * gv_xs_row(H) * 2; }
template <int QMASK, int S1, int MAXS, int NTHR>
__global__ __launch_bounds__(NTHR) void k_gv_gateup(GvArgs a) {
    constexpr int NW = NTHR / 64;
    __shared__ GvTables<QMASK, false> tb;
    __shared__ GvPair sp[GV_MAX_PAIRS];
    extern __shared__ u32x4 gv_xs[];
    const int tid = threadIdx.x;
    gv_load_pairs(a, sp);  // the pair table first: its loads are in flight while the rest is staged
    {
        const int units = a.H / 8, run = a.H / 128;  // 16-byte units per row and per lane run
        for (int i = tid; i < a.R * units; i += NTHR) {
            const int r = i / units, u = i - r * units;
            gv_xs[r * (gv_xs_row(a.H) / 8) + u + u / run] = reinterpret_cast<const u32x4*>(a.x)[i];
        }
    }
    tb.load(tid, NTHR);
    if (blockIdx.x == 0 && tid < FLAGS_WORDS) a.flags[tid] = 0;
    __syncthreads();
    if (blockIdx.x == 0 && tid < a.R * a.k) {
        a.pairs[tid] = sp[tid];
        if (sp[tid].e < 0) atomicOr(&a.flags[0], FLAG_BAD_ID);
    }
    const uint16_t* xs = reinterpret_cast<const uint16_t*>(gv_xs);
    const int lane = threadIdx.x & 63, rs = lane >> 4, q = lane & 15;
    const int half_i = a.I >> 1;
    const int total = a.R * a.k * half_i;
    const int span = a.H >> 4;
    for (int wv = blockIdx.x * NW + (threadIdx.x >> 6); wv < total; wv += gridDim.x * NW) {
        const int pr = wv / half_i;
        const int i0 = 2 * (wv % half_i);
        const int r = pr / a.k;
        const GvPair pp = sp[pr];
        const int e = pp.e;
        const int row = i0 + (rs & 1);
        float part = 0.f;
        if (e >= 0) {
            const uint8_t* W = a.arena + (rs < 2 ? pp.gate_off : pp.up_off);
            const uint32_t mb = (uint32_t)((size_t)a.I * a.H / 256 * (pp.qt == QT_T1 ? Fmt<QT_T1>::BYTES : Fmt<QT_Q2B>::BYTES));
            part = row_dot<QMASK, S1, MAXS, true>(pp.qt, W, mb, a.H, row, q * span, span,
                                                  xs + r * gv_xs_row(a.H) + q * (span + 8), tb);
        }
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
        const float other = __shfl_xor(part, 32, 64);  // gate lanes receive the up sum of their feature
        if (rs < 2 && q == 0)
            a.hgv[(size_t)pr * a.I + row] = f32_to_f16_bits(e >= 0 ? silu(part) * other : 0.f);
    }
}

// Work-groups per CU the down kernel below is built for: with both block types and one strip of
// at most 32 values per lane it needs just over 128 VGPRs; held to 128 (four waves per SIMD) a
// 2-row call's 4,096 waves (H = 2048) are resident at once instead of in two rounds.
template <int QMASK, int S2, int MAXS>
constexpr int gv_down_wgs() { return QMASK == 3 && MAXS == 1 && S2 <= 32 ? 4 : 1; }

// One wave per (row r, output column c): lane group gq = lane/16 takes slot j = 4*round + gq,
// each lane I/16 values of row c of that expert's W_down; after the 16-lane reduction the slot
// outputs are added to the accumulator in selection order j = 0..k-1.  The weights of all
// rounds are loaded before the first is decoded.
template <int QMASK, int S2, int MAXS, int NTHR>
__global__ __launch_bounds__(NTHR, (gv_down_wgs<QMASK, S2, MAXS>())) void k_gv_down(GvArgs a) {
    constexpr int NW = NTHR / 64;
    __shared__ GvTables<QMASK, true> tb;
    __shared__ GvPair sp[GV_MAX_PAIRS];
    __shared__ float wsh[GV_MAX_PAIRS];
    if (threadIdx.x < a.R * a.k) {
        sp[threadIdx.x] = a.pairs[threadIdx.x];  // resolved by the gate/up kernel
        wsh[threadIdx.x] = a.weight(threadIdx.x);
    }
    tb.load(threadIdx.x, NTHR);
    __syncthreads();
    const int lane = threadIdx.x & 63, gq = lane >> 4, q = lane & 15;
    const int span = a.I >> 4;
    const int nst = span / S2;
    constexpr int MAXR = GV_MAX_PAIRS / 2 / 4;  // rounds of 4 slots (k <= 16)
    for (int wv = blockIdx.x * NW + (threadIdx.x >> 6); wv < a.R * a.H; wv += gridDim.x * NW) {
        const int r = wv / a.H, c = wv % a.H;
        // loads of every round
        StripRaw<QT_T1, S2> rt[MAXR][MAXS];
        StripRaw<QT_Q2B, S2> rq[MAXR][MAXS];
#pragma unroll
        for (int rd = 0; rd < MAXR; ++rd) {
            const int j = 4 * rd + gq;
            if (4 * rd < a.k && j < a.k) {
                const GvPair p = sp[r * a.k + j];
                if (p.e >= 0) {
                    const uint32_t mb = (uint32_t)((size_t)a.I * a.H / 256 * (p.qt == QT_T1 ? Fmt<QT_T1>::BYTES : Fmt<QT_Q2B>::BYTES));
                    const BufSrc src(a.arena + p.down_off, mb);
#pragma unroll
                    for (int st = 0; st < MAXS; ++st)
                        if (st < nst) {
                            const uint32_t flat = (uint32_t)c * (uint32_t)a.I + (uint32_t)(q * span + st * S2);
                            if ((QMASK & 2) && (QMASK == 2 || p.qt == QT_T1))
                                rt[rd][st].load(src, (flat >> 8) * Fmt<QT_T1>::BYTES, (int)(flat & 255));
                            else if (QMASK & 1)
                                rq[rd][st].load(src, (flat >> 8) * Fmt<QT_Q2B>::BYTES, (int)(flat & 255));
                        }
                }
            }
        }
        float acc = 0.f;
#pragma unroll
        for (int rd = 0; rd < MAXR; ++rd) {
            const int j0 = 4 * rd;
            if (j0 >= a.k) break;
            const int j = j0 + gq;
            float part = 0.f;
            if (j < a.k) {
                const GvPair p = sp[r * a.k + j];
                if (p.e >= 0) {
                    const uint16_t* hx = a.hgv + (size_t)(r * a.k + j) * a.I + q * span;
#pragma unroll
                    for (int st = 0; st < MAXS; ++st)
                        if (st < nst) {
                            if constexpr (QMASK & 2) {
                                if (QMASK == 2 || p.qt == QT_T1) {
                                    part += strip_dot_raw<QT_T1, S2, false>(rt[rd][st], hx + st * S2, tb.t1);
                                    continue;
                                }
                            }
                            if constexpr (QMASK & 1) part += strip_dot_raw<QT_Q2B, S2, false>(rq[rd][st], hx + st * S2, tb.q2b);
                        }
                }
            }
#pragma unroll
            for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const float y = __shfl(part, 16 * s2, 64);
                if (j0 + s2 < a.k) acc = __fmaf_rn(wsh[r * a.k + j0 + s2], y, acc);
            }
        }
        if (lane == 0) a.out[(size_t)r * a.H + c] = a.res != nullptr ? acc + a.res[(size_t)r * a.H + c] : acc;
    }
}

// Four threads per block, each decoding a 64-value strip through the same decoder as the
// matrix kernels: out = (s*c) * block scale, exact in fp32.
template <int QT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ blocks, int64_t n_blocks,
                                                 float* __restrict__ out) {
    __shared__ DecodeTables<QT, false> tab;
    tab.build(threadIdx.x, 256);
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n_blocks * 4) return;
    const int64_t b = t >> 2;
    const int g = (int)(t & 3);
    // a buffer window of the single block (with its alignment preserved) keeps loads in bounds
    const uintptr_t base = (uintptr_t)(blocks + b * Fmt<QT>::BYTES);
    const uint32_t mis = (uint32_t)(base & 3);
    const uint8_t* b4 = (const uint8_t*)(base - mis);
    const BufSrc src(b4, mis + Fmt<QT>::BYTES);
    StripRaw<QT, 64> raw;
    raw.load(src, mis, 64 * g);
    Strip<QT, 64> st;
    st.prepare(raw, tab.tern);
    float* o = out + b * 256 + 64 * g;
    for (int f = 0; f < 8; ++f) {
        const u32x4 fr = st.frag(f, tab.val);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[8 * f + 2 * i] = __uint_as_float(fr[i] << 16) * st.d;
            o[8 * f + 2 * i + 1] = __uint_as_float(fr[i] & 0xFFFF0000u) * st.d;
        }
    }
}

// The MFMA operand decoders of the expert GEMMs (T1Dec8 on fp8 operands; Q2Dec16 on bf16 operands
// for gate/up, F16 = false, or fp16 operands for down, F16 = true), run exactly as the matrix
// kernels run them: the decoder tables built in LDS by GuTables, each block's window of dwords
// (from the dword boundary at or below the block start) in LDS, strip_prep with the block's byte
// misalignment, then every step's operands.  Lane (n, g) of a wave decodes lane group g's share of
// block 16 * wave_index + n and writes d * operand to the k position the operand byte (T1) or
// 16-bit half (Q2B) stands for (t1_kmap / q2_kmap).  d * operand is exact in fp32.
template <int QT, bool F16>
__global__ __launch_bounds__(256) void k_dequant_mfma(const uint8_t* __restrict__ base4, uint32_t mis,
                                                      int64_t n_blocks, float* __restrict__ out) {
    typedef GuTables<QT, F16> Tab;
    typedef WinGeo<QT> G;
    constexpr int WDW = G::WIN / 4;  // dwords per window
    __shared__ __attribute__((aligned(32768))) uint64_t t64[Tab::N64];
    __shared__ uint32_t tbl8[8];
    __shared__ uint32_t win[4][16][WDW];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
    Tab::build(t64, tbl8, tid, 256);
    const GuShared sh = Tab::shared(nullptr, nullptr, nullptr, t64, tbl8, nullptr, nullptr);
    const int64_t b0 = ((int64_t)blockIdx.x * 4 + wave) * 16;  // first block of this wave
    // the range of dwords that hold bytes of the blocks (reads beyond it return 0, as the matrix
    // kernels' windows past a matrix's last block do)
    const uint64_t span = (uint64_t)mis + (uint64_t)n_blocks * Fmt<QT>::BYTES;
    const BufSrc src(base4, (uint32_t)(span < 0xFFFFFFF0ull ? span : 0xFFFFFFF0ull));
    for (int i = lane; i < 16 * WDW; i += 64) {
        const int r = i / WDW, d = i % WDW;
        const int64_t b = b0 + r;
        uint32_t v = 0;
        if (b < n_blocks) v = src.dw(((uint32_t)(mis + (uint64_t)b * Fmt<QT>::BYTES) & ~3u) + 4u * (uint32_t)d);
        win[wave][r][d] = v;
    }
    __syncthreads();
    const int64_t b = b0 + n;
    if (b >= n_blocks) return;
    const uint32_t m = (uint32_t)(mis + (uint64_t)b * Fmt<QT>::BYTES) & 3u;
    T1Lane8 ln;
    ln.init(g);
    typename StripDec<QT>::type dec;
    strip_prep<QT>(dec, win[wave][n], m, g, ln, sh);
    float* o = out + b * 256;
    if constexpr (QT == QT_T1) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t op[8];
            dec.step(h, ln, sh.tsel, op);
#pragma unroll
            for (int p = 0; p < 32; ++p)
                o[t1_kmap(g, 32 * h + p)] = __builtin_amdgcn_cvt_f32_fp8((int)(op[p >> 2] >> (8 * (p & 3))), 0) * dec.d;
        }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                uint32_t op[8];
                dec.half(h, p, sh.qsel, op);
#pragma unroll
                for (int q = 0; q < 8; ++q) {  // dword q: operand 2p + q/4, values 2(q%4), 2(q%4)+1
                    const int j = 2 * p + (q >> 2);
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const uint32_t bits = (op[q] >> (16 * s)) & 0xFFFFu;
                        const float v = F16 ? half_bits_to_float(bits) : __uint_as_float(bits << 16);
                        o[q2_kmap(g, h, j, 2 * (q & 3) + s)] = v * dec.d;
                    }
                }
            }
    }
}

}  // namespace rl
