// Dispatch of a whole batch of at most kSmallAssign assignments by one
// workgroup of kSmallAssign threads: count, scan and rank in one pass.
//
// Page 3 (m.lsln.cn/news/228042), section "一个批次如何变成各专家专属的矩阵":
// the kept assignments are grouped per expert, each row keeping its source
// token; rows of an expert follow token order.
//
// Thread a owns assignment a. Lanes of a wave holding the same expert find
// each other by AND-ing one ballot per bit of the expert id, which gives each
// its rank among them; LDS turns the per-wave counts into wave prefixes per
// expert and the expert totals into offsets (exclusive scan). The resulting
// order is (expert, token), the same as the multi-workgroup path.
#pragma once

#include "moe_common.hpp"
#include "moe_internal.hpp"

namespace moe {

constexpr int kDispatchMaxE = 1024;
constexpr int kDispatchWaves = kSmallAssign / kWave;
static_assert(kDispatchMaxE == kSmallAssign, "the offsets scan takes one expert per thread");

struct DispatchSmem {
    int wc[kDispatchWaves][kDispatchMaxE];  // per-wave counts, then per-wave first rank
    int eoff[kDispatchMaxE];                // expert totals, then expert offsets
    int wsum[kDispatchWaves];
};

// All kSmallAssign threads of the workgroup must call this (it has barriers).
// ids/w: [n_assign] (w == 0: dropped); ebits: bits of E - 1 (0 for E == 1).
__device__ __forceinline__ void dispatch_whole(const int32_t* __restrict__ ids, const float* __restrict__ w,
                                               int n_assign, int k, int E, int ebits, int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ row_token, int32_t* __restrict__ inv,
                                               DispatchSmem& sm) {
    constexpr int NW = kDispatchWaves;
    const int tid = threadIdx.x, l = lane_id(), wv = tid / kWave;
    for (int i = tid; i < NW * E; i += kSmallAssign) sm.wc[i / E][i % E] = 0;
    const int a = tid;
    const bool valid = a < n_assign;
    const int id = valid ? ids[a] : 0;
    const bool kept = valid && w[a] != 0.0f && (unsigned)id < (unsigned)E;  // out-of-range ids: dropped
    const int e = kept ? id : 0;
    unsigned long long same = __ballot(kept);
    for (int b = 0; b < ebits; ++b) {
        const bool bit = (e >> b) & 1;
        const unsigned long long bal = __ballot(bit);
        same &= bit ? bal : ~bal;
    }
    const unsigned long long below = (l == 0) ? 0ull : (~0ull >> (kWave - l));
    const int rank = __popcll(same & below);
    const int cnt = __popcll(same);
    __syncthreads();
    if (kept && rank == 0) sm.wc[wv][e] = cnt;
    __syncthreads();
    for (int x = tid; x < E; x += kSmallAssign) {  // wave prefixes per expert, expert totals
        int run = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int c = sm.wc[i][x];
            sm.wc[i][x] = run;
            run += c;
        }
        sm.eoff[x] = run;
    }
    __syncthreads();
    const int v = tid < E ? sm.eoff[tid] : 0;
    const int incl = wave_incl_scan(v);
    if (l == kWave - 1) sm.wsum[wv] = incl;
    __syncthreads();
    int wbase = 0;
    for (int i = 0; i < wv; ++i) wbase += sm.wsum[i];
    const int excl = wbase + incl - v;
    if (tid < E) {
        sm.eoff[tid] = excl;
        offsets[tid] = excl;
    }
    if (tid == E - 1) offsets[E] = excl + v;
    __syncthreads();
    if (valid) {
        if (kept) {
            const int r = sm.eoff[e] + sm.wc[wv][e] + rank;
            row_token[r] = a / k;
            inv[a] = r;
        } else {
            inv[a] = -1;
        }
    }
}

__host__ __device__ inline int expert_bits(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

}  // namespace moe
