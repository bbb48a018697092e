// Router of the routed-expert layer (the step before it): fp32 router logits -> the k
// selected experts of every token and their renormalised weights.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "rl_kernels.h"

namespace rl {

// Router: one wave per token.  Lane l holds logits l, l + 64, ..., l + 64 (NR - 1) (NR = the
// power of two at or above E/64, at most 16); entries at or beyond E, and entries already
// selected, hold -inf (logits are finite, so -inf never wins while a real entry is left).
// Selection j takes the largest remaining logit, ties to the lower id: each lane offers its
// best remaining entry (scanned in ascending id with a strict comparison, so the lower id
// wins a tie) and an xor butterfly over (value descending, id ascending) leaves the winner in
// every lane; the lane that holds it replaces it by -inf.  Lane j keeps selection j.
// Weights: exp(l_j - max) over their sum taken in selection order (every lane adds the same
// k terms in the same order).
// One token's selection by one wave (logits lt[0..E-1]); lane j < k returns selection j: its
// expert id and renormalised weight.
template <int NR>
__device__ __forceinline__ void route_token(const float* __restrict__ lt, int E, int k, int lane, int& my_id,
                                            float& my_w) {
    float v[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int e = lane + 64 * r;
        const float x = lt[e < E ? e : E - 1];  // every load in bounds, all issued together
        v[r] = e < E ? x : -INFINITY;
    }
    my_id = 0;
    float my_v = 0.f, m = 0.f;
    for (int j = 0; j < k; ++j) {
        float bv = v[0];
        int bi = lane;
#pragma unroll
        for (int r = 1; r < NR; ++r) {
            const bool better = v[r] > bv;
            bv = better ? v[r] : bv;
            bi = better ? lane + 64 * r : bi;
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            const float ov = __shfl_xor(bv, d, 64);
            const int oi = __shfl_xor(bi, d, 64);
            const bool take = (ov > bv) | ((ov == bv) & (oi < bi));  // no short circuit: no branches
            bv = take ? ov : bv;
            bi = take ? oi : bi;
        }
#pragma unroll
        for (int r = 0; r < NR; ++r)
            if (bi == lane + 64 * r) v[r] = -INFINITY;
        if (lane == j) {
            my_id = bi;
            my_v = bv;
        }
        if (j == 0) m = bv;
    }
    const float ex = lane < k ? expf(my_v - m) : 0.f;
    float sum = 0.f;
    for (int j = 0; j < k; ++j) sum += __shfl(ex, j, 64);
    my_w = ex / sum;
}

template <int NR>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E, int k,
                                               int32_t* __restrict__ ids, float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (t >= T) return;  // uniform over the wave
    int id;
    float wt;
    route_token<NR>(logits + (size_t)t * E, E, k, lane, id, wt);
    if (lane < k) {
        ids[(size_t)t * k + lane] = id;
        w[(size_t)t * k + lane] = wt;
    }
}

// The router fused with the first launch of the pair grouping: work-groups [0, ntiles) each
// route the tokens of one grouping tile (g.tp / kk tokens, one wave per token at a time), write
// their topk_ids / topk_w and count the tile's pairs per expert in LDS (the shared expert's pair
// of every token included); the other work-groups split x (as k_count_split).  The grouping's
// scatter then reads the ids this launch wrote.
struct RouteArgs {
    const float* logits;  // [T][n_route]
    int32_t* ids;         // [T][k], written
    float* w;             // [T][k], written
    int T, n_route, k;
};

template <int NR, int LPR, int NG>
__global__ __launch_bounds__(256) void k_route_count_split(RouteArgs ra, GroupArgs g, SplitArgs a) {
    clear_words(g);
    if ((int)blockIdx.x >= g.ntiles) {
        split_rows<SPLIT_X, LPR, NG>(a, blockIdx.x - g.ntiles);
        return;
    }
    __shared__ int32_t h[MAX_E];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, tile = blockIdx.x;
    if (tile == 0 && tid < g.nflags) g.flags[tid] = 0;
    for (int e = tid; e < g.E; e += 256) h[e] = 0;
    __syncthreads();
    const int tpt = g.tp / g.pid.kk;  // tokens per tile
    const int t0 = tile * tpt, t1 = min(ra.T, t0 + tpt);
    for (int t = t0 + wave; t < t1; t += 4) {
        int id;
        float wt;
        route_token<NR>(ra.logits + (size_t)t * ra.n_route, ra.n_route, ra.k, lane, id, wt);
        if (lane < ra.k) {
            ra.ids[(size_t)t * ra.k + lane] = id;
            ra.w[(size_t)t * ra.k + lane] = wt;
            atomicAdd(&h[id], 1);
        }
    }
    if (g.pid.shared >= 0 && tid == 0 && t1 > t0) atomicAdd(&h[g.pid.shared], t1 - t0);
    __syncthreads();
    for (int e = tid; e < g.E; e += 256) g.tile_hist[(size_t)tile * g.E + e] = h[e];
}

}  // namespace rl
