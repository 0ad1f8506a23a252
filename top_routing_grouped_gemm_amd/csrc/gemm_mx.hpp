// Ragged grouped GEMM on MX fp8 operands (OCP microscaling: E4M3 codes, one
// power-of-two E8M0 scale per 32 consecutive values along the reduction axis)
// with v_mfma_scale_f32_32x32x64_f8f6f4, which applies both operands' block
// scales inside the matrix core.
//
// Operand lanes of the 32x32x64 form (fixed with an in-bounds probe): lane l
// holds row (A) or column (B) l%32; bytes 0..15 of its 32 belong to the 64-k
// slice's first 32-value block and bytes 16..31 to the second; lanes l and
// l+32 hold the two halves of each block, and the scale byte that lane l
// passes applies to block l/32 of its row or column. Here lane half h holds k
// = 16h..16h+15 of block 0 and 32+16h.. of block 1: two 16-byte runs.
//
// Stage layout (BK = 64 k, one MFMA slice): A [BM][64 B] and B [BN/128 tiles]
// [128][64 B], both with 16-byte chunk c of row r at c ^ f(r), f(r) =
// ((r >> 1) & 3) ^ ((r >> 3) & 1) (two 16-byte reads of 32 rows spread over
// the banks for 16- and 32-lane phases). A rows come either gathered from
// row-major token codes (64-byte pieces) or from a k-blocked code array
// [K/64][cap][64] (a stage of rows is one contiguous run); the loader applies
// the inverse XOR to the source. B tiles are copied verbatim (the quantiser
// pre-applies the XOR). Then one dword of 4 scale bytes (the 128-k block pair the stage
// belongs to) per A row and per B column, by 4-byte direct-to-LDS loads:
// waves 0..BM/64-1 load the A rows, the others the B columns, so every wave
// issues the same number of loads per stage. 34 KB stages, a 4-stage ring.
//
// Epilogue 3 re-quantises the SiLU output to MX along N (the next product's
// reduction axis): per row, each 32-column block's maximum comes from a
// 3-step xor shuffle after the quad transpose; the codes go to the k-blocked
// C[N/64][c_cap][64] the next launch reads as A, and the wave's four scale
// bytes (128 columns) to one dword of c_sc[N/128][c_cap][4].
#pragma once

#include "fp8_codes.hpp"
#include "gemm_dma.hpp"

namespace moe {
namespace dma {

constexpr int kMxBK = 64;
constexpr int kMxTileN = 128, kMxTileBytes = kMxTileN * kMxBK;  // 8 KiB weight code tiles
__host__ __device__ __forceinline__ int mx_swz(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

// One direct-to-LDS 4-byte load per lane: lane i's dword lands at lds_base + 4 * i.
__device__ __forceinline__ void lds_dma4(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_base), "v"(src) : "memory", "m0");
}

template <int TM, int TN, int WTM, int WTN>
__device__ __forceinline__ void store_tile_mx(f32x16 (&acc)[TM][TN], uint8_t* C, long c_cap,
                                              uint8_t* c_sc, int rb, int re, int n0, int N, int wm, int wn) {
    static_assert(WTN == 128 && TN == 4, "a wave's 128 columns give one scale dword per row");
    const int l = lane_id();
    const int c0 = (l & 31) & ~3, m = l & 3;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(C, (short)0, (int)((long)(N / kMxBK) * c_cap * kMxBK), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsc =
        __builtin_amdgcn_make_buffer_rsrc(c_sc, (short)0, (int)((long)(N / kMxTileN) * c_cap * 4), 0x00020000);
    const int colw = n0 + wn * WTN;  // a multiple of 128
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int rowrel = wm * WTM + i * 32 + 8 * p + 4 * (l >> 5) + m;
            const bool row_ok = rowrel < re - rb;
            uint32_t sdw = 0;
#pragma unroll
            for (int jj = 0; jj < TN; ++jj) {
                float v[4] = {acc[i][jj][4 * p], acc[i][jj][4 * p + 1], acc[i][jj][4 * p + 2], acc[i][jj][4 * p + 3]};
                quad_transpose(v);
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = silu_f32(v[q]);
                const float am = row32_absmax(v);  // this row's 32-column block
                const int x = mx_exponent(am);
                const uint32_t codes = mx_codes4(v[0], v[1], v[2], v[3], x);
                const int col = colw + jj * 32 + c0;
                const int off = (int)(((long)(col / kMxBK) * c_cap + rb + rowrel) * kMxBK + col % kMxBK);
                __builtin_amdgcn_raw_buffer_store_b32(codes, rs, (row_ok && col < N) ? off : 0x7ffffff0, 0, 0);
                sdw |= (uint32_t)(x + 127) << (8 * jj);
            }
            const bool w_ok = c0 == 0 && row_ok && colw < N;
            __builtin_amdgcn_raw_buffer_store_b32(
                sdw, rsc, w_ok ? (int)((((long)colw / kMxTileN) * c_cap + rb + rowrel) * 4) : 0x7ffffff0, 0, 0);
        }
}

// C[rows of group e, n-tile] = A[rows] @ B_e on MX operands.
//   A: the 64 codes of row r's k-block kb at A + kb*a_kstride + row(r)*a_rstride,
//      row(r) = a_rows[r] when gathering, else r (row-major: a_kstride = 64,
//      a_rstride = K; k-blocked [K/64][cap][64]: a_kstride = cap*64,
//      a_rstride = 64); scales a_sc + ((kb/2)*a_sc_rows + row(r))*4: the 4
//      bytes of the 128-k pair of blocks.
//   B: expert e's codes at B + e*strideB as 8 KiB tiles [Npad/128][K/64][128 n][64 k];
//      scales b_sc + e*b_sc_estride + ((kb/2)*Npad + n)*4.
//   EPI 1 / 4: fp32 / block-scaled fp16 as store_tile32 (ldc, c_cap); EPI 3: SiLU,
//   MX codes to the k-blocked C[N/64][c_cap][64] and scale dwords to c_sc[N/128][c_cap][4].
// Requirements (host): K % 128 == 0, K >= 128, N % 128 == 0.
template <int BM, int BN, int NS, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_mx_kernel(
    const uint8_t* __restrict__ A, long a_kstride, long a_rstride, const int32_t* __restrict__ a_rows,
    const uint8_t* __restrict__ a_sc, long a_sc_rows, const uint8_t* __restrict__ B,
    long strideB, const uint8_t* __restrict__ b_sc, long b_sc_estride, int Npad, void* __restrict__ C, long ldc,
    long c_cap, uint8_t* __restrict__ c_sc, const int32_t* __restrict__ offsets, int E, int rmin, int rmax, int N,
    int K, int n_tiles) {
    constexpr int NW = WM * WN, BK = kMxBK;
    constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, ASC = BM * 4, BSC = BN * 4;
    constexpr int STAGE = A_BYTES + B_BYTES + ASC + BSC;
    constexpr int A_CHUNKS = A_BYTES / (1024 * NW), B_CHUNKS = B_BYTES / (1024 * NW);
    constexpr int LOADS = A_CHUNKS + B_CHUNKS + 1;
    constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "whole KiB chunks per wave");
    static_assert(BM / 64 + BN / 64 == NW, "one scale load per wave");
    static_assert(BN % kMxTileN == 0 && NS * STAGE <= 160 * 1024, "shape");
    __shared__ __align__(1024) uint8_t smem[NS * STAGE];

    int e, rb, re, nt;
    if (!xcd_tile<BM>(offsets, E, 0, n_tiles, rmin, rmax, e, rb, re, nt)) return;
    const int n0 = nt * BN;
    const int wave = threadIdx.x / kWave, l = lane_id();
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const int KB = K / BK;

    const uint8_t* a_src[A_CHUNKS];
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        const int row = (uwave + NW * i) * 16 + l / 4;  // 16 rows of 64 bytes per KiB
        int grow = min(rb + row, re - 1);              // rows past the group repeat a valid row
        if (a_rows != nullptr) grow = a_rows[grow];
        a_src[i] = A + (long)grow * a_rstride + 16 * ((l % 4) ^ mx_swz(row));
    }
    const uint8_t* Be = B + (long)e * strideB;
    const int nb_last = Npad / kMxTileN - 1;
    const uint8_t* b_src[B_CHUNKS];
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
        const int c = uwave + NW * i;
        const int nb = min(n0 / kMxTileN + c / (kMxTileBytes / 1024), nb_last);
        b_src[i] = Be + (long)nb * KB * kMxTileBytes + (c % (kMxTileBytes / 1024)) * 1024 + 16 * l;
    }
    // scale dwords: waves 0..BM/64-1 take A rows 64w.., the others B columns
    const uint8_t* s_src;
    long s_kstep;  // bytes per 128-k block pair
    uint32_t s_dst;
    if (uwave < BM / 64) {
        int grow = min(rb + 64 * uwave + l, re - 1);
        if (a_rows != nullptr) grow = a_rows[grow];
        s_src = a_sc + (long)grow * 4;
        s_kstep = a_sc_rows * 4;
        s_dst = A_BYTES + B_BYTES + 256 * uwave;
    } else {
        const int col = min(n0 + 64 * (uwave - BM / 64) + l, Npad - 1);
        s_src = b_sc + (long)e * b_sc_estride + (long)col * 4;
        s_kstep = (long)Npad * 4;
        s_dst = A_BYTES + B_BYTES + ASC + 256 * (uwave - BM / 64);
    }
    lds_u8* ring = (lds_u8*)smem;
    auto issue = [&](int stage, int kb) {
        const uint32_t sb = (uint32_t)(uintptr_t)(ring + stage * STAGE);
        const uint32_t b0 = sb + uwave * 1024;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) lds_dma16(a_src[i] + (long)kb * a_kstride, b0 + i * 1024 * NW);
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i)
            lds_dma16(b_src[i] + (long)kb * kMxTileBytes, b0 + A_BYTES + i * 1024 * NW);
        lds_dma4(s_src + (long)(kb >> 1) * s_kstep, sb + s_dst);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    const int wm = uwave / WN, wn = uwave % WN, h = l >> 5;
    const bool active = rb + wm * WTM < re;
    auto compute = [&](lds_u8* St, int kb) {
        lds_u8* As = St;
        lds_u8* Bs = St + A_BYTES;
        lds_u8* Asc = St + A_BYTES + B_BYTES;
        lds_u8* Bsc = Asc + ASC;
        const int sh = 8 * (2 * (kb & 1) + h);  // this lane's 32-k block inside the 128-k scale dword
        i32x8 af[TM], bfr[TN];
        uint32_t sa[TM], sbv[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * WTM + i * 32 + (l & 31);
            lds_u8* base = As + row * BK;
            const u32x4 lo = *(lds_u32x4*)(base + 16 * (h ^ mx_swz(row)));
            const u32x4 hi = *(lds_u32x4*)(base + 16 * ((2 + h) ^ mx_swz(row)));
            af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                          (int)hi[3]};
            sa[i] = (*(lds_u32*)(Asc + row * 4) >> sh) & 0xffu;
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = wn * WTN + j * 32 + (l & 31);
            const int nn = n % kMxTileN;
            lds_u8* base = Bs + (n / kMxTileN) * kMxTileBytes + nn * BK;
            const u32x4 lo = *(lds_u32x4*)(base + 16 * (h ^ mx_swz(nn)));
            const u32x4 hi = *(lds_u32x4*)(base + 16 * ((2 + h) ^ mx_swz(nn)));
            bfr[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                           (int)hi[3]};
            sbv[j] = (*(lds_u32*)(Bsc + n * 4) >> sh) & 0xffu;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], acc[i][j], 0, 0, 0,
                                                                            (int)sa[i], 0, (int)sbv[j]);
    };

    const int nsteps = K / BK;  // >= 2
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < nsteps) issue(s, s);
    for (int s = 0; s < nsteps; ++s) {
        wait_stage<LOADS, NS - 2>(min(NS - 2, nsteps - 1 - s));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (s + NS - 1 < nsteps) issue((s + NS - 1) % NS, s + NS - 1);
        __builtin_amdgcn_sched_barrier(0);
        if (active) compute(ring + (s % NS) * STAGE, s);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (!active) return;
    if constexpr (EPI == 3)
        store_tile_mx<TM, TN, WTM, WTN>(acc, (uint8_t*)C, c_cap, c_sc, rb, re, n0, N, wm, wn);
    else  // buffer ranges over this tile's rows only
        store_tile32<TM, TN, WTM, WTN, EPI>(acc, C, ldc, c_cap, rb, min(re, rb + BM), n0, N, wm, wn);
}

// EPI 3 for waves of 32 columns: SiLU, one 32-value block per row and wave,
// its codes as one dword and its scale as one byte of the row's 128-column
// scale dword (waves of a workgroup own distinct bytes of it).
template <int TM>
__device__ __forceinline__ void store_tile_mx32(f32x16 (&acc)[TM][1], uint8_t* C, long c_cap, uint8_t* c_sc, int rb,
                                                int re, int colw, int N, int wm, int wtm) {
    const int l = lane_id();
    const int c0 = (l & 31) & ~3, m = l & 3;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(C, (short)0, (int)((long)(N / kMxBK) * c_cap * kMxBK), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsc =
        __builtin_amdgcn_make_buffer_rsrc(c_sc, (short)0, (int)((long)(N / kMxTileN) * c_cap * 4), 0x00020000);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int rowrel = wm * wtm + i * 32 + 8 * p + 4 * (l >> 5) + m;
            const bool ok = rowrel < re - rb && colw < N;
            float v[4] = {acc[i][0][4 * p], acc[i][0][4 * p + 1], acc[i][0][4 * p + 2], acc[i][0][4 * p + 3]};
            quad_transpose(v);
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = silu_f32(v[q]);
            const float am = row32_absmax(v);  // this row's 32-column block
            const int x = mx_exponent(am);
            const uint32_t codes = mx_codes4(v[0], v[1], v[2], v[3], x);
            const int col = colw + c0;
            const int off = (int)(((long)(col / kMxBK) * c_cap + rb + rowrel) * kMxBK + col % kMxBK);
            __builtin_amdgcn_raw_buffer_store_b32(codes, rs, ok ? off : 0x7ffffff0, 0, 0);
            const int soff = (int)((((long)colw / kMxTileN) * c_cap + rb + rowrel) * 4 + (colw % kMxTileN) / 32);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(x + 127), rsc, (ok && c0 == 0) ? soff : 0x7ffffff0, 0, 0);
        }
}

// Weight-streaming MX shape for few rows per group (decode): one 32-row MFMA
// block against a 128-column weight slab, 4 waves of 32 columns, 128-k stages
// (two 64-k MX products per stage: A pieces of 128 bytes, B two adjacent 8 KiB
// code tiles, read non-temporally since each slab is read once), NS-stage
// ring. Operand and scale layouts, requirements and epilogues as
// gemm_mx_kernel; per stage each wave issues one A chunk, four B chunks and
// one 4-byte scale load (wave 0: the 32 rows' A scales; waves 1, 2: B
// columns 0-63, 64-127; wave 3 repeats wave 2's into a spare slot).
template <int NS, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_mx_stream_kernel(
    const uint8_t* __restrict__ A, long a_kstride, long a_rstride, const int32_t* __restrict__ a_rows,
    const uint8_t* __restrict__ a_sc, long a_sc_rows, const uint8_t* __restrict__ B, long strideB,
    const uint8_t* __restrict__ b_sc, long b_sc_estride, int Npad, void* __restrict__ C, long ldc, long c_cap,
    uint8_t* __restrict__ c_sc, const int32_t* __restrict__ offsets, int E, int rmin, int rmax, int N, int K,
    int n_tiles) {
    constexpr int BM = 32, BN = kMxTileN, BK2 = 2 * kMxBK, NW = 4;
    constexpr int A_BYTES = BM * BK2, B_BYTES = BN * BK2, SC = 256;  // scale slots: A, B 0-63, B 64-127, spare
    constexpr int STAGE = A_BYTES + B_BYTES + 4 * SC;
    constexpr int LOADS = 1 + 4 + 1;
    static_assert(A_BYTES == 1024 * NW && B_BYTES == 4 * 1024 * NW, "one A and four B KiB chunks per wave");
    static_assert(NS * STAGE <= 160 * 1024, "LDS");
    __shared__ __align__(1024) uint8_t smem[NS * STAGE];

    int e, rb, re, nt;
    if (!xcd_tile<BM>(offsets, E, 0, n_tiles, rmin, rmax, e, rb, re, nt)) return;
    const int n0 = nt * BN;
    const int wave = threadIdx.x / kWave, l = lane_id();
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const int KB = K / kMxBK;

    // A chunk of this wave: rows 8*uwave + l/8, 16-byte piece l%8 of the 128-k slice (pieces 0-3 from the
    // first 64-k block, 4-7 from the second), placed at piece position (l%8) ^ swz(row) of a 128-byte row
    const int arow = 8 * uwave + l / 8;
    int grow = min(rb + arow, re - 1);  // rows past the group repeat a valid row
    if (a_rows != nullptr) grow = a_rows[grow];
    const int apiece = (l % 8) ^ ((arow >> 1) & 7);
    const uint8_t* a_src = A + (long)(apiece / 4) * a_kstride + (long)grow * a_rstride + 16 * (apiece % 4);
    // B chunks: the stage's two tiles are 16 KiB contiguous; chunk c = uwave + 4i
    const uint8_t* Be = B + (long)e * strideB;
    const int nb = min(n0 / kMxTileN, Npad / kMxTileN - 1);
    const uint8_t* b_src = Be + (long)nb * KB * kMxTileBytes + uwave * 1024 + 16 * l;
    // scale dwords
    const uint8_t* s_src;
    long s_kstep;
    if (uwave == 0) {
        int srow = min(rb + (l & 31), re - 1);
        if (a_rows != nullptr) srow = a_rows[srow];
        s_src = a_sc + (long)srow * 4;
        s_kstep = a_sc_rows * 4;
    } else {
        const int col = min(n0 + 64 * min(uwave - 1, 1) + l, Npad - 1);
        s_src = b_sc + (long)e * b_sc_estride + (long)col * 4;
        s_kstep = (long)Npad * 4;
    }
    lds_u8* ring = (lds_u8*)smem;
    auto issue = [&](int stage, int kp) {  // kp: 128-k step
        const uint32_t sb = (uint32_t)(uintptr_t)(ring + stage * STAGE);
        lds_dma16(a_src + (long)(2 * kp) * a_kstride, sb + uwave * 1024);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lds_dma16_nt(b_src + (long)(2 * kp) * kMxTileBytes + i * 4096, sb + A_BYTES + (uwave + 4 * i) * 1024);
        lds_dma4(s_src + (long)kp * s_kstep, sb + A_BYTES + B_BYTES + SC * uwave);
    };

    f32x16 acc[1][1];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[0][0][q] = 0.f;
    const int h = l >> 5;
    auto compute = [&](lds_u8* St) {
        lds_u8* As = St;
        lds_u8* Bs = St + A_BYTES;
        lds_u8* Asc = St + A_BYTES + B_BYTES;
        lds_u8* Bsc = Asc + SC;  // columns 0-127 in the two B slots
        const int row = l & 31, n = uwave * 32 + (l & 31);
        const uint32_t sa_dw = *(lds_u32*)(Asc + row * 4);
        const uint32_t sb_dw = *(lds_u32*)(Bsc + n * 4);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            lds_u8* abase = As + row * BK2;
            const u32x4 alo = *(lds_u32x4*)(abase + 16 * ((4 * kk + h) ^ ((row >> 1) & 7)));
            const u32x4 ahi = *(lds_u32x4*)(abase + 16 * ((4 * kk + 2 + h) ^ ((row >> 1) & 7)));
            lds_u8* bbase = Bs + kk * kMxTileBytes + n * kMxBK;
            const u32x4 blo = *(lds_u32x4*)(bbase + 16 * (h ^ mx_swz(n)));
            const u32x4 bhi = *(lds_u32x4*)(bbase + 16 * ((2 + h) ^ mx_swz(n)));
            const i32x8 af = {(int)alo[0], (int)alo[1], (int)alo[2], (int)alo[3],
                              (int)ahi[0], (int)ahi[1], (int)ahi[2], (int)ahi[3]};
            const i32x8 bf = {(int)blo[0], (int)blo[1], (int)blo[2], (int)blo[3],
                              (int)bhi[0], (int)bhi[1], (int)bhi[2], (int)bhi[3]};
            const int sh = 8 * (2 * kk + h);
            acc[0][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, acc[0][0], 0, 0, 0,
                                                                        (int)((sa_dw >> sh) & 0xffu), 0,
                                                                        (int)((sb_dw >> sh) & 0xffu));
        }
    };

    const int nsteps = K / BK2;  // >= 1
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < nsteps) issue(s, s);
    for (int s = 0; s < nsteps; ++s) {
        wait_stage<LOADS, NS - 2>(min(NS - 2, nsteps - 1 - s));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (s + NS - 1 < nsteps) issue((s + NS - 1) % NS, s + NS - 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(ring + (s % NS) * STAGE);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (EPI == 3)
        store_tile_mx32<1>(acc, (uint8_t*)C, c_cap, c_sc, rb, re, n0 + 32 * uwave, N, 0, BM);
    else  // buffer ranges over this tile's rows only
        store_tile32<1, 1, BM, 32, EPI>(acc, C, ldc, c_cap, rb, min(re, rb + BM), n0, N, 0, uwave);
}

}  // namespace dma
}  // namespace moe
