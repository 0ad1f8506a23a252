// Wave-wide top-k pieces shared by the router and the capacity-limited
// selection. One wave holds one token's E <= 64*Q logits, lane l holding
// experts l, l+64, ... so that ascending expert id is q-major order.
//
// Page 1 ("MoE大模型的智能调度…", www.jsqmd.com/news/1091713), section 2.2,
// routing layer: keep the top-k logits, softmax them into weights, zero a
// weight below the threshold and renormalise.
#pragma once

#include <float.h>
#include <math.h>

#include "moe_common.hpp"

namespace moe {

// Order-preserving map of a float to an unsigned key (larger float, larger
// key). Callers add +0.0f first so that -0 and +0 get the same key (equal
// logits tie); key 0 lies below every real logit and marks "not a candidate".
__device__ __forceinline__ uint32_t ord_key(float v) {
    const uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// The k largest keys of the wave, ties to the lower expert id:
//  1. radix select: the k-th largest key tau is built bit by bit from the
//     top, keeping a bit when at least k keys are >= the candidate (a wave
//     ballot and a popcount per slice; no cross-lane shuffles). With EARLY,
//     a candidate with exactly k keys >= it ends the walk: those keys are
//     the k largest and no tie can straddle the k-th place;
//  2. keys > tau are selected; keys == tau fill the remaining places in
//     ascending expert id.
// EARLY pays two scalar instructions per bit for the shorter walk: it helps
// where few waves run the select (capacity rounds on the skewed workload:
// 173 -> 150 us) and costs where many do, since the walk is scalar-bound
// there (prefill reduction 7.4 -> 8.2 us).
// Needs at least k keys > 0.
template <int Q, bool EARLY = false>
__device__ __forceinline__ void radix_select(const uint32_t (&key)[Q], int k, bool (&sel)[Q]) {
    const int l = lane_id();
    uint32_t tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = tau | (1u << bit);
        int c = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) c += __popcll(__ballot(key[q] >= cand));
        if (EARLY && c == k) {  // wave-uniform (ballot counts)
#pragma unroll
            for (int q = 0; q < Q; ++q) sel[q] = key[q] >= cand;
            return;
        }
        if (c >= k) tau = cand;
    }
    int n_gt = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) n_gt += __popcll(__ballot(key[q] > tau));
    const int need = k - n_gt;  // >= 1 places left for keys equal to tau
    const unsigned long long below = (1ull << l) - 1ull;
    int ties = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const unsigned long long m = __ballot(key[q] == tau);
        const int before = ties + __popcll(m & below);
        sel[q] = key[q] > tau || (key[q] == tau && before < need);
        ties += __popcll(m);
    }
}

// Softmax over the selected logits, then the optional drop (w < drop -> 0)
// and renormalisation. p: weights of the selected entries, 0 elsewhere.
template <int Q>
__device__ __forceinline__ void softmax_drop(const float (&v)[Q], const bool (&sel)[Q], float drop, float (&p)[Q],
                                             bool (&kept)[Q]) {
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < Q; ++q)
        if (sel[q]) mx = fmaxf(mx, v[q]);
    mx = wave_max(mx);
    float ps = 0.0f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        p[q] = sel[q] ? expf(v[q] - mx) : 0.0f;
        ps += p[q];
    }
    const float sum = wave_sum(ps);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        p[q] = p[q] / sum;
        kept[q] = sel[q];
    }
    if (drop > 0.0f) {
        float ks = 0.0f;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            kept[q] = sel[q] && !(p[q] < drop);
            if (!kept[q]) p[q] = 0.0f;
            ks += p[q];
        }
        const float kept_sum = wave_sum(ks);
#pragma unroll
        for (int q = 0; q < Q; ++q) p[q] = p[q] / kept_sum;
    }
}

// Slot of a selected expert = rank of its id among the selected (ballot
// prefix counts). Writes ids[t*k + slot] and, when wout is not null, the
// weight (a kept weight clamped to >= FLT_MIN so that 0.0f always means
// dropped).
template <int Q>
__device__ __forceinline__ void write_slots(const bool (&sel)[Q], const bool (&kept)[Q], const float (&p)[Q], long t,
                                            int k, int32_t* __restrict__ ids, float* __restrict__ wout) {
    const int l = lane_id();
    const unsigned long long below = (1ull << l) - 1ull;
    int base = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const unsigned long long m = __ballot(sel[q]);
        if (sel[q]) {
            const int slot = base + __popcll(m & below);
            ids[t * k + slot] = q * kWave + l;
            if (wout != nullptr) wout[t * k + slot] = kept[q] ? fmaxf(p[q], FLT_MIN) : 0.0f;
        }
        base += __popcll(m);
    }
}

}  // namespace moe
