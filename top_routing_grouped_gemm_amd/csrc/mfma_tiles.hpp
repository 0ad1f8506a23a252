// LDS staging of bf16 operand tiles for the v_mfma_f32_16x16x32_bf16 matrix
// core instruction on gfx950.
//
// The instruction multiplies a 16x32 A block by a 32x16 B block. Each lane
// feeds eight consecutive-k bf16 values of one A row (row = lane % 16) and
// eight of one B column (column = lane % 16), from k-slice lane / 16; it
// returns four fp32 results of column lane % 16, rows 4*(lane/16) .. +3.
// Both operands therefore want k-contiguous LDS rows: A tiles are stored
// [m][k] as they come from memory; B tiles, which are n-contiguous in memory
// (W1[E,H,F], W2[E,F,H], Wr[H,E]), are transposed on their way into LDS and
// stored [n][k]. Rows are padded by 8 bf16 (16 bytes) to spread LDS banks.
#pragma once

#include "moe_common.hpp"

namespace moe {

// Copy rows [r_begin, r_end) x cols [k0, k0+BK) of a row-major bf16 matrix
// (leading dimension lda, K columns, K % 8 == 0) into dst[m][k] (row stride
// S elements), zero-filling rows past r_end and columns past K. Tile row m
// maps to matrix row r_begin + m; BM tile rows in total.
template <int BM, int BK, int NT>
__device__ __forceinline__ void load_a_tile_regs(const uint16_t* __restrict__ A, long lda, int r_begin, int r_end,
                                                 int K, int k0, u32x4 (&reg)[(BM * BK / 8 + NT - 1) / NT]) {
    constexpr int KV = BK / 8;
    constexpr int N = (BM * BK / 8 + NT - 1) / NT;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int idx = threadIdx.x + i * NT;
        const int m = idx / KV, kv = idx % KV;
        const int r = r_begin + m, kk = k0 + kv * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (idx < BM * KV && r < r_end && kk < K) v = *(const u32x4*)(A + (long)r * lda + kk);
        reg[i] = v;
    }
}

template <int BM, int BK, int NT, int S>
__device__ __forceinline__ void store_a_tile_lds(uint16_t* dst, const u32x4 (&reg)[(BM * BK / 8 + NT - 1) / NT]) {
    constexpr int KV = BK / 8;
    constexpr int N = (BM * BK / 8 + NT - 1) / NT;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int idx = threadIdx.x + i * NT;
        if (idx < BM * KV) {
            const int m = idx / KV, kv = idx % KV;
            *(u32x4*)(dst + m * S + kv * 8) = reg[i];
        }
    }
}

// B tile: rows [k0, k0+BK) x cols [n0, n0+BN) of a row-major bf16 [K x N]
// matrix (leading dimension ldb; N % 8 == 0, ldb % 8 == 0). Each work item is
// a 4(k) x 8(n) block: four 16-byte loads that are transposed in registers
// into eight 8-byte k-runs, one per n.
template <int BK, int BN, int NT>
struct BTile {
    static constexpr int ITEMS = (BK / 4) * (BN / 8);
    static constexpr int PER_THREAD = (ITEMS + NT - 1) / NT;
    u32x4 r[PER_THREAD][4];

    __device__ __forceinline__ void load(const uint16_t* __restrict__ B, long ldb, int K, int N, int k0, int n0) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int idx = threadIdx.x + i * NT;
            const int nv = idx % (BN / 8), kb = idx / (BN / 8);
            const int n = n0 + nv * 8;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int kk = k0 + kb * 4 + q;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (idx < ITEMS && n < N && kk < K) v = *(const u32x4*)(B + (long)kk * ldb + n);
                r[i][q] = v;
            }
        }
    }

    template <int S>
    __device__ __forceinline__ void store(uint16_t* dst) const {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int idx = threadIdx.x + i * NT;
            if (idx >= ITEMS) continue;
            const int nv = idx % (BN / 8), kb = idx / (BN / 8);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int wsel = c >> 1;
                const bool hi = c & 1;
                uint32_t e0 = hi ? (r[i][0][wsel] >> 16) : (r[i][0][wsel] & 0xFFFFu);
                uint32_t e1 = hi ? (r[i][1][wsel] >> 16) : (r[i][1][wsel] & 0xFFFFu);
                uint32_t e2 = hi ? (r[i][2][wsel] >> 16) : (r[i][2][wsel] & 0xFFFFu);
                uint32_t e3 = hi ? (r[i][3][wsel] >> 16) : (r[i][3][wsel] & 0xFFFFu);
                u32x2 pk = {e0 | (e1 << 16), e2 | (e3 << 16)};
                *(u32x2*)(dst + (nv * 8 + c) * S + kb * 4) = pk;
            }
        }
    }
};

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const uint16_t* a_row, const uint16_t* b_row, f32x4 acc) {
    const bf16x8 a = *(const bf16x8*)a_row;
    const bf16x8 b = *(const bf16x8*)b_row;
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

}  // namespace moe
