// Router of the routed-expert layer (the step before it): fp32 router logits -> the k
// selected experts of every token and their renormalised weights.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

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

}  // namespace rl
