// Ragged grouped GEMM mainloop built on two gfx950 data paths:
//
//  * direct-to-LDS 16-byte global loads (global_load_lds_dwordx4): each
//    lane's 16 bytes land at LDS base + 16 * lane, so one wave instruction
//    fills a contiguous 1 KiB LDS chunk without touching VGPRs, and several
//    LDS stages can be in flight at once;
//  * the LDS transpose read ds_read_b64_tr_b16: within each 16-lane group,
//    lane j supplies the address of a 4-element row j of a 16x4 block of
//    16-bit values and lane i receives elements [4q + i/4][i%4], q = 0..3.
//    With lane j pointing at B[kb + j/4][n0 + 4*(j%4)], lane i receives
//    B[kb + q][n0 + i]: four k-consecutive values of column n0 + i, which is
//    the k-packed B operand of v_mfma_f32_16x16x32_bf16. B tiles therefore
//    stay n-contiguous in LDS, exactly as W1[E,H,F] and W2[E,F,H] lie in HBM.
//
// LDS layouts are XOR-swizzled at 16-byte granularity so that the operand
// reads of one instruction spread over all banks:
//   A [BM][BK=64] (128 B rows):  chunk c of row r sits at c ^ ((r >> 1) & 7)
//   B [BK][BN]    (2*BN B rows): chunk c of row r sits at c ^ fB(r), where
//                 fB(r) = 2 * ((r & 3) + 4 * ((r >> 3) & 1)) keeps 32-byte
//                 pairs together and separates the rows one read touches.
// The loader applies the inverse permutation to the global addresses it
// fetches, so every global row segment is still read contiguously.
//
// The router (route.hip) uses the same loader, swizzles and transpose reads
// with 16x16x32 MFMAs; the grouped FFN uses gemm32_kernel below.
//
// Tile order is XCD-aware: workgroups are dealt to the 8 XCDs round-robin,
// so workgroup b runs on XCD b % 8; the ragged tile sequence (experts in
// order, M-tiles of an expert in order, N-tiles fastest) is cut into 8
// contiguous chunks and XCD x walks chunk x. Workgroups that share an
// expert's weight slab or an A tile then share one L2.
#pragma once

#include "moe_common.hpp"

namespace moe {
namespace dma {

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

constexpr int kXcds = 8;

// s_waitcnt immediate that waits for vmcnt <= n and leaves the other counters free (gfx9 encoding).
template <int N>
struct VmWait {
    static constexpr int value = (N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14);
};
// vmcnt <= n and lgkmcnt == 0 (every LDS read of this wave has returned).
template <int N>
struct VmLgkmWait {
    static constexpr int value = (N & 15) | (7 << 4) | (((N >> 4) & 3) << 14);
};

// Wait until at most `ahead` later stages of LOADS loads each are still in
// flight (loads complete in issue order), with all LDS reads returned.
// s_waitcnt takes an immediate, hence the unrolled ladder over ahead = MAXA..0.
template <int LOADS, int MAXA>
__device__ __forceinline__ void wait_stage(int ahead) {
    static_assert(MAXA * LOADS <= 63, "vmcnt is 6 bits");
    if constexpr (MAXA == 0) {
        __builtin_amdgcn_s_waitcnt(VmLgkmWait<0>::value);
    } else {
        if (ahead >= MAXA) __builtin_amdgcn_s_waitcnt(VmLgkmWait<MAXA * LOADS>::value);
        else wait_stage<LOADS, MAXA - 1>(ahead);
    }
}

// One direct-to-LDS 16-byte load per lane: lane i's 16 bytes from `src` land
// at LDS byte address lds_base + 16 * i (lds_base wave-uniform, via M0).
// Issued from inline asm so that the compiler does not track it as an LDS
// write: the kernel orders it with its own s_waitcnt vmcnt + s_barrier, and
// the main loop has no other vector-memory operation whose waits it could
// disturb (vmcnt decrements in issue order, so extra loads in flight only
// make any compiler-placed wait stricter).
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(src) : "memory", "m0");
}

// The same load with the non-temporal cache policy: for weights a launch
// streams once (the few-row shapes read every expert slab exactly once), so
// they do not displace reused lines. Measured at decode: grouped FFN 126 ->
// 112 us (bf16), 71 -> 66 us (fp8 codes).
__device__ __forceinline__ void lds_dma16_nt(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds_base), "v"(src) : "memory", "m0");
}

__device__ __forceinline__ int swz_a(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }
__device__ __forceinline__ int swz_b(int row, int chunk) { return chunk ^ (2 * ((row & 3) + 4 * ((row >> 3) & 1))); }

// Map this workgroup to (expert, M-tile rows, N-tile). All waves compute the
// same answer; returns false for workgroups past the last tile. Only groups
// with rmin <= rows < rmax get tiles (another launch takes the others).
// extra_rows > 0 (with offsets only): one more group of that many rows after
// the E groups, reported as e_out == E with rows [0, extra_rows) of its own.
template <int BM>
__device__ __forceinline__ bool xcd_tile_lanes(const int32_t* __restrict__ offsets, int E, int fixed_rows,
                                               int n_tiles, int rmin, int rmax, int& e_out, int& rb, int& re, int& nt,
                                               int extra_rows) {
    const int l = lane_id();
    int total_m, incl = 0, s = 0, per = 1;
    if (offsets == nullptr) {
        total_m = (fixed_rows + BM - 1) / BM;
    } else {
        per = (E + kWave - 1) / kWave;
        const int e0 = l * per, e1 = min(E, e0 + per);
        for (int e = e0; e < e1; ++e) {
            const int c = offsets[e + 1] - offsets[e];
            s += (c >= rmin && c < rmax) ? (c + BM - 1) / BM : 0;
        }
        incl = wave_incl_scan(s);
        total_m = __shfl(incl, kWave - 1, kWave);
    }
    const int grouped_m = total_m;
    total_m += (extra_rows + BM - 1) / BM;
    const long total = (long)total_m * n_tiles;
    const long chunk = (total + kXcds - 1) / kXcds;
    const long b = blockIdx.x;
    if (b >= chunk * kXcds) return false;
    const long t = (b % kXcds) * chunk + b / kXcds;
    if (t >= total) return false;
    const int mt = (int)(t / n_tiles);
    nt = (int)(t % n_tiles);
    if (offsets == nullptr) {
        e_out = 0;
        rb = mt * BM;
        re = min(fixed_rows, rb + BM);
        return true;
    }
    if (mt >= grouped_m) {
        e_out = E;
        rb = (mt - grouped_m) * BM;
        re = min(extra_rows, rb + BM);
        return true;
    }
    const unsigned long long own = __ballot(mt < incl);
    const int L = __ffsll((long long)own) - 1;
    int before = __shfl(incl - s, L, kWave);
    const int eL0 = L * per, eL1 = min(E, eL0 + per);
    int e = eL0;
    for (; e < eL1; ++e) {
        const int c = offsets[e + 1] - offsets[e];
        const int tt = (c >= rmin && c < rmax) ? (c + BM - 1) / BM : 0;
        if (mt < before + tt) break;
        before += tt;
    }
    e_out = e;
    rb = offsets[e] + (mt - before) * BM;
    re = min(offsets[e + 1], rb + BM);
    return true;
}

// The tile is the same for every lane; saying so keeps it, and the pointers
// and buffer descriptors derived from it, in scalar registers (otherwise each
// epilogue buffer store is wrapped in a loop over distinct descriptor values).
template <int BM>
__device__ __forceinline__ bool xcd_tile(const int32_t* __restrict__ offsets, int E, int fixed_rows, int n_tiles,
                                         int rmin, int rmax, int& e_out, int& rb, int& re, int& nt,
                                         int extra_rows = 0) {
    e_out = rb = re = nt = 0;
    const bool ok = xcd_tile_lanes<BM>(offsets, E, fixed_rows, n_tiles, rmin, rmax, e_out, rb, re, nt, extra_rows);
    e_out = __builtin_amdgcn_readfirstlane(e_out);
    rb = __builtin_amdgcn_readfirstlane(rb);
    re = __builtin_amdgcn_readfirstlane(re);
    nt = __builtin_amdgcn_readfirstlane(nt);
    return __builtin_amdgcn_readfirstlane((int)ok) != 0;
}

// C[rows of group e, n-tile] = A[rows] @ B_e with the fused epilogue, on
// v_mfma_f32_32x32x16_bf16 (in a bare loop as fast as the 16x16x32 form, with
// half as many instructions for the same wave tile).
// Requirements (checked on the host): K % BK == 0, K >= 2*BK, N % 8 == 0,
// lda % 8 == 0, ldb % 8 == 0.
//
// Workgroup: WM x WN waves (8 by default: two per SIMD, which doubles the
// number of direct-to-LDS loads in flight per CU; one wave's 16-byte loads
// alone cap the L2-to-LDS feed near 12 TB/s chip-wide). Each wave owns a
// (BM/WM) x (BN/WN) block of 32x32 accumulators.
//
// 32x32x16 operand and result lanes: A lane l holds row l%32, k-slice
// 8*(l/32)..+7; B lane l holds column l%32 and the same k-slice, built from
// two transpose reads (16-lane group G covers columns 16*(G&1)..+15 of the
// tile and k-half G>>1); result lane l holds column l%32, rows
// 8*(q/4) + 4*(l/32) + q%4 for q = 0..15.
//
// Pipeline: a ring of NS LDS stages of BK k-values. k-step s waits (s_waitcnt
// vmcnt) for its own loads, meets the other waves at a fence-free s_barrier
// (after which every wave has landed step s and finished reading the stage of
// step s-1), starts the loads of step s+NS-1 into that freed stage, then runs
// its MFMAs, so NS-1 stages of loads are always in flight.
__device__ __forceinline__ int swz_b32(int r, int c) { return c ^ (4 * (r & 3)); }

template <int BK>
__device__ __forceinline__ int swz_a32(int r, int c) {
    if constexpr (BK == 64) return c ^ ((r >> 1) & 7);  // 128-byte rows, 8 chunks
    else return c ^ ((r >> 2) & 3);                     // 64-byte rows, 4 chunks
}

// Epilogue helpers of the 32x32 kernel.
__device__ __forceinline__ float dpp_swap1(float v) {  // lane i <- lane i^1 within quads
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_swap2(float v) {  // lane i <- lane i^2 within quads
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Largest |v| over the 32 columns of one row after quad_transpose: the lanes
// holding them share l % 4 and l / 32 (8 quads). Rotations by 4 and 8 lanes
// inside each 16-lane DPP row, then an exchange with the other 16-lane row of
// the same 32-lane half (permlane16 swap); all of it on the VALU, no LDS
// round trips. Compared as integers: non-negative floats order like their
// bit patterns.
__device__ __forceinline__ float row32_absmax(const float (&v)[4]) {
    int b = max(max(__float_as_int(v[0]) & 0x7fffffff, __float_as_int(v[1]) & 0x7fffffff),
                max(__float_as_int(v[2]) & 0x7fffffff, __float_as_int(v[3]) & 0x7fffffff));
    b = max(b, __builtin_amdgcn_mov_dpp(b, 0x124, 0xF, 0xF, false));  // row_ror:4
    b = max(b, __builtin_amdgcn_mov_dpp(b, 0x128, 0xF, 0xF, false));  // row_ror:8
    const auto s = __builtin_amdgcn_permlane16_swap((unsigned)b, (unsigned)b, false, false);
    return __int_as_float(max((int)s[0], (int)s[1]));
}

// 4x4 transpose across the 4 lanes of a quad: on entry lane m holds column m
// (v[r] = M[r][m]); on exit it holds row m (v[c] = M[m][c]).
__device__ __forceinline__ void quad_transpose(float (&v)[4]) {
    const int m = lane_id() & 3;
    const bool o1 = m & 1, o2 = m & 2;
    float s0 = o1 ? v[0] : v[1], s1 = o1 ? v[2] : v[3];
    float r0 = dpp_swap1(s0), r1 = dpp_swap1(s1);
    float y0 = o1 ? r0 : v[0], y1 = o1 ? v[1] : r0, y2 = o1 ? r1 : v[2], y3 = o1 ? v[3] : r1;
    s0 = o2 ? y0 : y2;
    s1 = o2 ? y1 : y3;
    r0 = dpp_swap2(s0);
    r1 = dpp_swap2(s1);
    v[0] = o2 ? r0 : y0;
    v[1] = o2 ? r1 : y1;
    v[2] = o2 ? y2 : r0;
    v[3] = o2 ? y3 : r1;
}

// Writes a workgroup's accumulators for rows [rb, re) and columns n0.. of C
// (re at most rb + the tile's rows, so the byte ranges below stay small):
// a quad transpose gives each lane 4 adjacent columns of one row, stored with
// one 16-byte (fp32) or 8-byte (SiLU + bf16) buffer store. Rows past the group
// and columns past N get an out-of-range offset and are dropped by the buffer
// descriptor, so no store sits behind a branch and every lane issues the same
// number of stores.
//
// c_cap > 0 selects the k-blocked layout [N/32][c_cap][32] for C (N % 32 == 0,
// N * c_cap * element bytes < 2^31): element (r, n) at ((n/32)*c_cap + r)*32
// + n%32. Consecutive rows of one 32-column block are then adjacent, so the
// next GEMM's A-tile loads of 32 k-values over consecutive rows are one
// contiguous run instead of 64-byte pieces of separate rows. Rows past the
// group are dropped by an explicit out-of-range offset in that layout.
//
// EPI 4 (fp32 result as block-scaled fp16, for a result read once more): per
// row and 32-column block a power of two 2^s puts the block's largest
// magnitude in [2^14, 2^15) (s = floor(log2 max) - 14, clamped to
// [-127, 127]; s = 0 for an all-zero block); the values v * 2^-s rounded to
// fp16 (nearest even; relative error <= 2^-11, absolute <= 2^(s-25) for the
// values under fp16's normal range; no overflow for any finite input) go to
// C[r*ldc + n] (2-byte elements) and s as a signed byte to
// (C + c_cap*ldc*2)[r*(ldc/32) + n/32], c_cap being the row capacity:
// 2 + 1/32 bytes per value instead of 4 (N % 32 == 0, ldc % 32 == 0).
template <int TM, int TN, int WTM, int WTN, int EPI>
__device__ __forceinline__ void store_tile32(f32x16 (&acc)[TM][TN], void* C, long ldc, long c_cap, int rb, int re,
                                             int n0, int N, int wm, int wn) {
    if constexpr (EPI == 4) {
        const int l = lane_id();
        const int lds = (int)(ldc / 32);  // scale bytes per row
        const __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc(
            (uint8_t*)C + ((long)rb * ldc + n0) * 2, (short)0, (int)(((long)(re - rb) * ldc - n0) * 2), 0x00020000);
        const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
            (uint8_t*)C + c_cap * ldc * 2 + (long)rb * lds + n0 / 32, (short)0, (int)((long)(re - rb) * lds - n0 / 32),
            0x00020000);
        const int c0 = (l & 31) & ~3, m = l & 3;
        // a wave spanning whole 128-column groups (n0 and ldc multiples of 128) gathers the 4 scale bytes
        // of each group in a register and stores them as one aligned 4-byte word; otherwise byte stores
        constexpr bool kWord = TN % 4 == 0;
        const bool word = kWord && ldc % 128 == 0 && n0 % 128 == 0;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int rowrel = wm * WTM + i * 32 + 8 * p + 4 * (l >> 5) + m;
                uint32_t sw = 0;
#pragma unroll
                for (int jj = 0; jj < TN; ++jj) {
                    const int blk = wn * WTN + jj * 32;     // first column of this 32-column block, tile-relative
                    const bool col_ok = n0 + blk + c0 < N;  // this lane's 4 columns (N % 32 == 0: whole blocks)
                    float v[4] = {acc[i][jj][4 * p], acc[i][jj][4 * p + 1], acc[i][jj][4 * p + 2],
                                  acc[i][jj][4 * p + 3]};
                    quad_transpose(v);
                    if (!col_ok) v[0] = v[1] = v[2] = v[3] = 0.0f;
                    const float am = row32_absmax(v);
                    const int ex = (int)((__float_as_uint(am) >> 23) & 0xffu);
                    const int sc = am > 0.0f ? min(127, max(-127, ex - 127 - 14)) : 0;
                    uint32_t hbits[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const _Float16 h = (_Float16)ldexpf(v[q], -sc);
                        hbits[q] = (uint32_t)__builtin_bit_cast(uint16_t, h);
                    }
                    typedef __attribute__((ext_vector_type(2))) unsigned u2;
                    const u2 pk = {hbits[0] | (hbits[1] << 16), hbits[2] | (hbits[3] << 16)};
                    const int e = rowrel * (int)ldc + blk + c0;  // element offset within the tile's rows
                    __builtin_amdgcn_raw_buffer_store_b64(pk, rs_v, col_ok ? e * 2 : 0x7ffffff0, 0, 0);
                    if (kWord) sw |= (uint32_t)(uint8_t)(int8_t)sc << (8 * (jj & 3));
                    if (!word)
                        __builtin_amdgcn_raw_buffer_store_b8(
                            (uint8_t)(int8_t)sc, rs_s, (col_ok && c0 == 0) ? rowrel * lds + blk / 32 : 0x7ffffff0, 0,
                            0);
                    if (kWord && (jj & 3) == 3) {
                        const int blk0 = blk - 96;  // the group's first block
                        if (word)
                            __builtin_amdgcn_raw_buffer_store_b32(
                                sw, rs_s, (c0 == 0 && n0 + blk0 < N) ? rowrel * lds + blk0 / 32 : 0x7ffffff0, 0, 0);
                        sw = 0;
                    }
                }
            }
        return;
    }
    constexpr int ES = EPI == 0 ? 2 : 4;
    const int l = lane_id();
    const long ldc_b = ldc * ES;
    const bool blocked = c_cap > 0;
    const __amdgpu_buffer_rsrc_t rsrc =
        blocked ? __builtin_amdgcn_make_buffer_rsrc(C, (short)0, (int)((long)N * c_cap * ES), 0x00020000)
                : __builtin_amdgcn_make_buffer_rsrc((uint8_t*)C + (long)rb * ldc_b + (long)n0 * ES, (short)0,
                                                    (int)((long)(re - rb) * ldc_b - (long)n0 * ES), 0x00020000);
    const int c0 = (l & 31) & ~3, m = l & 3;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) {
            const int colrel = wn * WTN + jj * 32 + c0;
            const bool col_ok = n0 + colrel < N;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float v[4] = {acc[i][jj][4 * p], acc[i][jj][4 * p + 1], acc[i][jj][4 * p + 2], acc[i][jj][4 * p + 3]};
                quad_transpose(v);
                const int rowrel = wm * WTM + i * 32 + 8 * p + 4 * (l >> 5) + m;
                int off;
                if (blocked)
                    off = (col_ok && rowrel < re - rb)
                              ? (int)((((long)(n0 + colrel - c0) >> 5) * c_cap + rb + rowrel) * (32 * ES) + c0 * ES)
                              : 0x7ffffff0;
                else
                    off = col_ok ? rowrel * (int)ldc_b + colrel * ES : 0x7ffffff0;
                if (EPI == 0) {
                    typedef __attribute__((ext_vector_type(2))) unsigned u2;
                    const u2 pk = {pack_bf16x2(silu_f32(v[0]), silu_f32(v[1])),
                                   pack_bf16x2(silu_f32(v[2]), silu_f32(v[3]))};
                    __builtin_amdgcn_raw_buffer_store_b64(pk, rsrc, off, 0, 0);
                } else {
                    const f32x4 pk = {v[0], v[1], v[2], v[3]};
                    __builtin_amdgcn_raw_buffer_store_b128(pk, rsrc, off, 0, 0);
                }
            }
        }
}

// The same stores for accumulators of the swapped product: with the weight
// fragment as the MFMA's first operand and the activation fragment as its
// second, block (i, j) holds the transposed 32x32 result, so lane l owns row
// wm*WTM + i*32 + l%32 and, in acc[i][j][4p..4p+3], the 4 adjacent columns
// wn*WTN + j*32 + 8p + 4*(l/32) + 0..3. No cross-lane transpose is needed, and
// the 32 columns of a row's block sit in lanes l and l^32 (EPI 4's block
// maximum is 15 local maxima and one permlane32 swap). Same layouts, ranges
// and dropped stores as store_tile32.
template <int TM, int TN, int WTM, int WTN, int EPI>
__device__ __forceinline__ void store_tile32s(f32x16 (&acc)[TM][TN], void* C, long ldc, long c_cap, int rb, int re,
                                              int n0, int N, int wm, int wn) {
    const int l = lane_id();
    const int h4 = 4 * (l >> 5);
    if constexpr (EPI == 4) {
        const int lds = (int)(ldc / 32);  // scale bytes per row
        const __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc(
            (uint8_t*)C + ((long)rb * ldc + n0) * 2, (short)0, (int)(((long)(re - rb) * ldc - n0) * 2), 0x00020000);
        const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
            (uint8_t*)C + c_cap * ldc * 2 + (long)rb * lds + n0 / 32, (short)0, (int)((long)(re - rb) * lds - n0 / 32),
            0x00020000);
        constexpr bool kWord = TN % 4 == 0;
        const bool word = kWord && ldc % 128 == 0 && n0 % 128 == 0;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int rowrel = wm * WTM + i * 32 + (l & 31);
            uint32_t sw = 0;
#pragma unroll
            for (int jj = 0; jj < TN; ++jj) {
                const int blk = wn * WTN + jj * 32;  // first column of this 32-column block, tile-relative
                const bool col_ok = n0 + blk < N;    // N % 32 == 0: whole blocks
                int b = 0;
#pragma unroll
                for (int q = 0; q < 16; ++q) b = max(b, __float_as_int(acc[i][jj][q]) & 0x7fffffff);
                const auto sx = __builtin_amdgcn_permlane32_swap((unsigned)b, (unsigned)b, false, false);
                b = col_ok ? max((int)sx[0], (int)sx[1]) : 0;
                const float am = __int_as_float(b);
                const int ex = (int)((__float_as_uint(am) >> 23) & 0xffu);
                const int sc = am > 0.0f ? min(127, max(-127, ex - 127 - 14)) : 0;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    uint32_t hbits[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const _Float16 h = (_Float16)ldexpf(acc[i][jj][4 * p + q], -sc);
                        hbits[q] = (uint32_t)__builtin_bit_cast(uint16_t, h);
                    }
                    typedef __attribute__((ext_vector_type(2))) unsigned u2;
                    const u2 pk = {hbits[0] | (hbits[1] << 16), hbits[2] | (hbits[3] << 16)};
                    const int e = rowrel * (int)ldc + blk + 8 * p + h4;  // element offset within the tile's rows
                    __builtin_amdgcn_raw_buffer_store_b64(pk, rs_v, col_ok ? e * 2 : 0x7ffffff0, 0, 0);
                }
                // the row's scale byte: lane l < 32 (lane l + 32 holds the other half of the same row)
                if (kWord) sw |= (uint32_t)(uint8_t)(int8_t)sc << (8 * (jj & 3));
                if (!word)
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(int8_t)sc, rs_s,
                                                         (col_ok && l < 32) ? rowrel * lds + blk / 32 : 0x7ffffff0, 0,
                                                         0);
                if (kWord && (jj & 3) == 3) {
                    const int blk0 = blk - 96;  // the group's first block
                    if (word)
                        __builtin_amdgcn_raw_buffer_store_b32(
                            sw, rs_s, (l < 32 && n0 + blk0 < N) ? rowrel * lds + blk0 / 32 : 0x7ffffff0, 0, 0);
                    sw = 0;
                }
            }
        }
        return;
    }
    constexpr int ES = EPI == 0 ? 2 : 4;
    const long ldc_b = ldc * ES;
    const bool blocked = c_cap > 0;
    const __amdgpu_buffer_rsrc_t rsrc =
        blocked ? __builtin_amdgcn_make_buffer_rsrc(C, (short)0, (int)((long)N * c_cap * ES), 0x00020000)
                : __builtin_amdgcn_make_buffer_rsrc((uint8_t*)C + (long)rb * ldc_b + (long)n0 * ES, (short)0,
                                                    (int)((long)(re - rb) * ldc_b - (long)n0 * ES), 0x00020000);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int rowrel = wm * WTM + i * 32 + (l & 31);
#pragma unroll
        for (int jj = 0; jj < TN; ++jj)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int colrel = wn * WTN + jj * 32 + 8 * p + h4;
                const bool col_ok = n0 + colrel < N;  // N % 8 == 0: all 4 columns or none
                int off;
                if (blocked)
                    off = (col_ok && rowrel < re - rb)
                              ? (int)((((long)(n0 + colrel) >> 5) * c_cap + rb + rowrel) * (32 * ES) +
                                      ((n0 + colrel) & 31) * ES)
                              : 0x7ffffff0;
                else
                    off = col_ok ? rowrel * (int)ldc_b + colrel * ES : 0x7ffffff0;
                const float v[4] = {acc[i][jj][4 * p], acc[i][jj][4 * p + 1], acc[i][jj][4 * p + 2],
                                    acc[i][jj][4 * p + 3]};
                if (EPI == 0) {
                    typedef __attribute__((ext_vector_type(2))) unsigned u2;
                    const u2 pk = {pack_bf16x2(silu_f32(v[0]), silu_f32(v[1])),
                                   pack_bf16x2(silu_f32(v[2]), silu_f32(v[3]))};
                    __builtin_amdgcn_raw_buffer_store_b64(pk, rsrc, off, 0, 0);
                } else {
                    const f32x4 pk = {v[0], v[1], v[2], v[3]};
                    __builtin_amdgcn_raw_buffer_store_b128(pk, rsrc, off, 0, 0);
                }
            }
    }
}

// The stores of store_tile32s through LDS, for a wave tile WTN = 128 columns
// wide: the same values, layouts and dropped stores, but each store
// instruction writes whole lines (fp32 row-major: 2 rows x 512 bytes; SiLU +
// bf16 k-blocked: 16 consecutive rows x 64 bytes of one 32-column block;
// block-scaled fp16: 2 rows x 256 bytes) instead of 16 or 32 bytes on each
// of 16 or 32 lines, which a CU issues several times as
// fast: per-workgroup timestamps put the fp32 epilogue of a 256 x 256 tile at
// 5.0 against 8.5-9.4 us. Launches gain less (about 1 % per layer), because
// the faster stores now compete with the next tiles' loads.
// Each wave stages its own 32 x 128 block (one i at a time) in its own LDS
// region `st` (16 KiB) with the pieces of row r XOR-permuted by a function of
// r, so that in each pass of the LDS (128 bytes: 16 lanes of 8-byte or 8 of
// 16-byte accesses) the writes (rows at one column) and the reads (pieces of
// whole rows) touch distinct banks. The caller has made the region free (every wave past
// the main loop's LDS reads). Supported: EPI 1 row-major, EPI 0 k-blocked,
// EPI 4 (its scale bytes are stored directly, as in store_tile32s).
template <int TM, int TN, int WTM, int WTN, int EPI>
__device__ __forceinline__ void store_tile32s_lds(f32x16 (&acc)[TM][TN], void* C, long ldc, long c_cap, int rb,
                                                  int re, int n0, int N, int wm, int wn, lds_u8* st) {
    static_assert(WTN == 128 && TN == 4 && kWave == 64, "32 x 128 staged blocks");
    static_assert(EPI == 0 || EPI == 1 || EPI == 4, "staged epilogues");
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    typedef __attribute__((ext_vector_type(2))) unsigned u2;
    typedef __attribute__((address_space(3))) u2 lds_u2;
    const int l = lane_id();
    const int r = l & 31, hl = l >> 5;
    if constexpr (EPI == 1) {
        // rows of 32 chunks of 16 bytes, chunk c of row r at c ^ r
        const long ldc_b = ldc * 4;
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (uint8_t*)C + (long)rb * ldc_b + (long)n0 * 4, (short)0, (int)((long)(re - rb) * ldc_b - (long)n0 * 4),
            0x00020000);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int c = 8 * j + 2 * p + hl;  // this lane's 4 columns, in 16-byte chunks
                    const f32x4 v = {acc[i][j][4 * p], acc[i][j][4 * p + 1], acc[i][j][4 * p + 2],
                                     acc[i][j][4 * p + 3]};
                    *(lds_f32x4*)(st + (r * 32 + (c ^ r)) * 16) = v;
                }
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int rr = 2 * k + hl, q = l & 31;
                const f32x4 v = *(lds_f32x4*)(st + (rr * 32 + (q ^ rr)) * 16);
                const int rowrel = wm * WTM + i * 32 + rr, colrel = wn * WTN + 4 * q;
                const int off = n0 + colrel < N ? rowrel * (int)ldc_b + colrel * 4 : 0x7ffffff0;
                __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, off, 0, 0);
            }
        }
    } else if constexpr (EPI == 0) {
        // k-blocked C: staged as [block j][row][32 columns], 8-byte piece g of row r at g ^ ((r >> 1) & 7)
        // (of the XOR functions measured, the one with the fewest bank conflicts: about 0.3 % of the
        // launch's CU-cycles, against 0.6 % with (r >> 2) & 7)
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(C, (short)0, (int)((long)N * c_cap * 2),
                                                                               0x00020000);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int g = 2 * p + hl;
                    const u2 pk = {pack_bf16x2(silu_f32(acc[i][j][4 * p]), silu_f32(acc[i][j][4 * p + 1])),
                                   pack_bf16x2(silu_f32(acc[i][j][4 * p + 2]), silu_f32(acc[i][j][4 * p + 3]))};
                    *(lds_u2*)(st + (j * 32 + r) * 64 + (g ^ ((r >> 1) & 7)) * 8) = pk;
                }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int j = k >> 1, rr = (k & 1) * 16 + (l >> 2), q = l & 3, f = (rr >> 1) & 7;
                const u2 lo = *(lds_u2*)(st + (j * 32 + rr) * 64 + ((2 * q) ^ f) * 8);
                const u2 hi = *(lds_u2*)(st + (j * 32 + rr) * 64 + ((2 * q + 1) ^ f) * 8);
                const int rowrel = wm * WTM + i * 32 + rr, col = n0 + wn * WTN + j * 32;
                const int off = (col < N && rowrel < re - rb)
                                    ? (int)((((long)col >> 5) * c_cap + rb + rowrel) * 64 + q * 16)
                                    : 0x7ffffff0;
                typedef __attribute__((ext_vector_type(4))) unsigned u4;
                const u4 v = {lo[0], lo[1], hi[0], hi[1]};
                __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, off, 0, 0);
            }
        }
    } else {
        // block-scaled fp16: values staged row-major [row][128 columns], 8-byte piece g of row r at g ^ r
        const int lds_sc = (int)(ldc / 32);  // scale bytes per row
        const __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc(
            (uint8_t*)C + ((long)rb * ldc + n0) * 2, (short)0, (int)(((long)(re - rb) * ldc - n0) * 2), 0x00020000);
        const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
            (uint8_t*)C + c_cap * ldc * 2 + (long)rb * lds_sc + n0 / 32, (short)0,
            (int)((long)(re - rb) * lds_sc - n0 / 32), 0x00020000);
        const bool word = ldc % 128 == 0 && n0 % 128 == 0;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int rowrel = wm * WTM + i * 32 + r;
            uint32_t sw = 0;
#pragma unroll
            for (int jj = 0; jj < TN; ++jj) {
                const int blk = wn * WTN + jj * 32;
                const bool col_ok = n0 + blk < N;
                int b = 0;
#pragma unroll
                for (int q = 0; q < 16; ++q) b = max(b, __float_as_int(acc[i][jj][q]) & 0x7fffffff);
                const auto sx = __builtin_amdgcn_permlane32_swap((unsigned)b, (unsigned)b, false, false);
                b = col_ok ? max((int)sx[0], (int)sx[1]) : 0;
                const float am = __int_as_float(b);
                const int ex = (int)((__float_as_uint(am) >> 23) & 0xffu);
                const int sc = am > 0.0f ? min(127, max(-127, ex - 127 - 14)) : 0;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    uint32_t hbits[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const _Float16 h = (_Float16)ldexpf(acc[i][jj][4 * p + q], -sc);
                        hbits[q] = (uint32_t)__builtin_bit_cast(uint16_t, h);
                    }
                    const u2 pk = {hbits[0] | (hbits[1] << 16), hbits[2] | (hbits[3] << 16)};
                    const int g = 8 * jj + 2 * p + hl;
                    *(lds_u2*)(st + r * 256 + (g ^ r) * 8) = pk;
                }
                sw |= (uint32_t)(uint8_t)(int8_t)sc << (8 * (jj & 3));
                if (!word)
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(int8_t)sc, rs_s,
                                                         (col_ok && l < 32) ? rowrel * lds_sc + blk / 32 : 0x7ffffff0,
                                                         0, 0);
            }
            if (word)
                __builtin_amdgcn_raw_buffer_store_b32(
                    sw, rs_s, (l < 32 && n0 + wn * WTN < N) ? rowrel * lds_sc + (wn * WTN) / 32 : 0x7ffffff0, 0, 0);
            // 8 bytes per lane, so that the 16 lanes of an LDS pass read 16 distinct banks' pieces of one row;
            // each store still writes 2 whole rows of 256 bytes
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int rr = 2 * k + (l >> 5), pc = l & 31;
                const u2 v = *(lds_u2*)(st + rr * 256 + (pc ^ rr) * 8);
                const int rrel = wm * WTM + i * 32 + rr, colrel = wn * WTN + 4 * pc;
                const int off = n0 + colrel < N ? (rrel * (int)ldc + colrel) * 2 : 0x7ffffff0;
                __builtin_amdgcn_raw_buffer_store_b64(v, rs_v, off, 0, 0);
            }
        }
    }
}

// fp8 B operand (F8B): expert weights as OCP e4m3 codes in 8 KiB tiles of
// 128 output columns x 64 k, laid out [N/128][K/64][128 n][64 k] per expert,
// with the 8-byte k-chunk c of column n stored at chunk c ^ f8_swz(n). A
// stage then copies whole tiles verbatim; a B fragment (8 k-consecutive codes
// of one column) is one ds_read_b64, and the swizzle spreads the 32 columns a
// read touches over distinct bank groups both for 16- and for 32-lane phases.
constexpr int kF8TileN = 128, kF8TileK = 64, kF8TileBytes = kF8TileN * kF8TileK;
__host__ __device__ __forceinline__ int f8_swz(int n) { return ((n >> 1) & 7) ^ ((n >> 4) & 1); }

template <int BM, int BN, int BK, int NS, int WM, int WN, bool F8B = false>
struct Tile32 {
    static constexpr int NW = WM * WN;
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * (F8B ? 1 : 2), STAGE = A_BYTES + B_BYTES;
    static constexpr int A_CHUNKS = A_BYTES / (1024 * NW), B_CHUNKS = B_BYTES / (1024 * NW);
    static constexpr int LOADS = A_CHUNKS + B_CHUNKS;          // vm ops per lane per stage
    static constexpr int A_RCH = BK / 8, A_RPK = 1024 / (BK * 2);
    static constexpr int B_RCH = BN / 8, B_RPK = 1024 / (BN * 2);
    static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
    static_assert(TM >= 1 && TN >= 1, "wave tile");
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "whole KiB chunks per wave");
    static_assert(BN * 2 <= 1024 && BK * 2 <= 1024 && (BK == 32 || BK == 64), "row sizes");
    static_assert(BN >= 128, "swz_b32 XORs chunk indices with up to 12: rows need >= 16 chunks of 8 columns");
    static_assert(!F8B || (BK == kF8TileK && BN % kF8TileN == 0), "fp8 B stages are whole 128 x 64 tiles");
    static_assert(NS * STAGE <= 160 * 1024, "LDS");
};

// One more group of a grouped launch with operands of its own: the shared
// expert (every token, read from x directly, its own weight matrix and
// output). rows == 0: none. Its tiles follow the E groups' tiles.
struct ExtraGroup {
    const uint16_t* A;  // A of its rows 0..rows-1, same conventions as the kernel's A
    long lda, a_kstep;
    const void* B;      // one weight matrix (no expert stride)
    void* C;            // its output, same conventions as the kernel's C
    long ldc, c_cap;
    int rows;
};

// a_rows (nullable): A row of output row r is a_rows[r] (the permute folded
// into the A-tile loads: A is then x[T,H] and a_rows the row -> token map).
// A element (r, k) sits at A[r*lda + (k/BK)*BK*a_kstep + k%BK]: row-major is
// lda = K, a_kstep = 1; the k-blocked layout written by store_tile32 with
// c_cap = cap is lda = 32, a_kstep = cap (BK == 32 only).
// c_cap: 0 for a row-major C with leading dimension ldc, else the k-blocked C.
// F8B: B holds the fp8 tiles described at f8_swz (strideB in bytes per
// expert, ldb unused) and bscale[e*N + n] the fp32 scale of column n of
// expert e, applied to the fp32 accumulators before the epilogue. The codes
// widen exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8, scale 1), so the MFMAs
// are the bf16 ones and sum_k a*code is exact up to fp32 accumulation.
// xg: the extra group (bf16 B only), stored with epilogue EPI2.
// With bf16 B the weight fragment is the MFMA's first operand and the results
// are stored by store_tile32s (no transpose; measured 1-2 % faster per launch
// at prefill, bit-identical results); the fp8 path keeps the activation first,
// so each lane's accumulators share one column and one weight scale.
template <int BM, int BN, int BK, int NS, int WM, int WN, int EPI, bool F8B = false, int EPI2 = EPI>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm32_kernel(const uint16_t* __restrict__ A, long lda,
                                                                 long a_kstep, const int32_t* __restrict__ a_rows,
                                                                 const void* __restrict__ B, long strideB, long ldb,
                                                                 const float* __restrict__ bscale,
                                                                 void* __restrict__ C, long ldc, long c_cap,
                                                                 const int32_t* __restrict__ offsets, int E,
                                                                 int fixed_rows, int rmin, int rmax, int N, int K,
                                                                 int n_tiles, ExtraGroup xg) {
    using Tl = Tile32<BM, BN, BK, NS, WM, WN, F8B>;
    constexpr int NW = Tl::NW, TM = Tl::TM, TN = Tl::TN, WTM = Tl::WTM, WTN = Tl::WTN;
    constexpr int A_BYTES = Tl::A_BYTES, STAGE = Tl::STAGE, LOADS = Tl::LOADS;
    constexpr bool SWP = !F8B;
    __shared__ __align__(1024) uint8_t smem[NS * STAGE];

    int e, rb, re, nt;
    if (!xcd_tile<BM>(offsets, E, fixed_rows, n_tiles, rmin, rmax, e, rb, re, nt, F8B ? 0 : xg.rows)) return;
    const int n0 = nt * BN;
    const bool extra = !F8B && e == E;
    if (extra) {
        A = xg.A;
        lda = xg.lda;
        a_kstep = xg.a_kstep;
        a_rows = nullptr;
        C = xg.C;
        ldc = xg.ldc;
        c_cap = xg.c_cap;
    }
    const uint8_t* Be = extra ? (const uint8_t*)xg.B : (const uint8_t*)B + (long)e * strideB * (F8B ? 1 : 2);
    const int wave = threadIdx.x / kWave, l = lane_id();
    const int uwave = __builtin_amdgcn_readfirstlane(wave);

    // global source of each LDS chunk this lane fills (inverse XOR = same XOR)
    const uint16_t* a_src[Tl::A_CHUNKS];
#pragma unroll
    for (int i = 0; i < Tl::A_CHUNKS; ++i) {
        const int c = uwave + NW * i;
        const int row = c * Tl::A_RPK + l / Tl::A_RCH;
        int grow = min(rb + row, re - 1);  // rows past the group repeat a valid row
        if (a_rows != nullptr) grow = a_rows[grow];
        a_src[i] = A + (long)grow * lda + swz_a32<BK>(row, l % Tl::A_RCH) * 8;
    }
    const uint8_t* b_src[Tl::B_CHUNKS];
    long b_kbytes;  // bytes of B per unit of k0
    if constexpr (F8B) {
        const int nb_last = (N + kF8TileN - 1) / kF8TileN - 1;
#pragma unroll
        for (int i = 0; i < Tl::B_CHUNKS; ++i) {
            const int c = uwave + NW * i;  // KiB chunk of the stage's B tiles
            const int nb = min(n0 / kF8TileN + c / (kF8TileBytes / 1024), nb_last);  // tiles past N repeat the last
            b_src[i] = Be + (long)nb * (K / kF8TileK) * kF8TileBytes + (c % (kF8TileBytes / 1024)) * 1024 + 16 * l;
        }
        b_kbytes = kF8TileBytes / kF8TileK;
    } else {
#pragma unroll
        for (int i = 0; i < Tl::B_CHUNKS; ++i) {
            const int c = uwave + NW * i;
            const int row = c * Tl::B_RPK + l / Tl::B_RCH;
            const int col = min(n0 + swz_b32(row, l % Tl::B_RCH) * 8, N - 8);  // columns past N repeat a valid chunk
            b_src[i] = Be + ((long)row * ldb + col) * 2;
        }
        b_kbytes = ldb * 2;
    }
    lds_u8* ring = (lds_u8*)smem;
    auto issue = [&](int stage, int k0) {
        const uint32_t b0 = (uint32_t)(uintptr_t)(ring + stage * STAGE) + uwave * 1024;
#pragma unroll
        for (int i = 0; i < Tl::A_CHUNKS; ++i) lds_dma16(a_src[i] + (long)k0 * a_kstep, b0 + i * 1024 * NW);
#pragma unroll
        for (int i = 0; i < Tl::B_CHUNKS; ++i) {
            // few-row tiles (BM <= 32) stream each weight slab once: non-temporal
            if constexpr (BM <= 32) lds_dma16_nt(b_src[i] + (long)k0 * b_kbytes, b0 + A_BYTES + i * 1024 * NW);
            else lds_dma16(b_src[i] + (long)k0 * b_kbytes, b0 + A_BYTES + i * 1024 * NW);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    const int wm = uwave / WN, wn = uwave % WN;
    // A wave whose 64 rows all lie past the group's end (the ragged last M-tile
    // of a group) skips its LDS reads, MFMAs and stores but keeps its share of
    // the loads and barriers. Waves w and w+4 share a SIMD and cover opposite
    // row halves, so a tile with <= BM/2 valid rows runs in about half the time.
    const bool active = rb + wm * WTM < re;
    auto read_frags = [&](lds_u8* As, int ks, bf16x8 (&af)[TM], bf16x8 (&bfr)[TN]) {
        lds_u8* Bs = As + A_BYTES;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * WTM + i * 32 + (l & 31);
            af[i] = *(lds_bf16x8*)(As + row * (BK * 2) + swz_a32<BK>(row, (ks >> 3) + (l >> 5)) * 16);
        }
        if constexpr (F8B) {
            typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
            typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
            const int kc = (ks >> 3) + (l >> 5);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = wn * WTN + j * 32 + (l & 31);
                const int nn = n % kF8TileN;
                const u32x2 q = *(lds_u32x2*)(Bs + (n / kF8TileN) * kF8TileBytes + nn * kF8TileK +
                                              ((kc ^ f8_swz(nn)) << 3));
                const bf16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, false);
                const bf16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, true);
                const bf16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, false);
                const bf16x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, true);
                typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
                const bf16x4 lo = __builtin_shufflevector(b0, b1, 0, 1, 2, 3);
                const bf16x4 hi = __builtin_shufflevector(b2, b3, 0, 1, 2, 3);
                bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            return;
        }
        const int G = l >> 4, j4 = l & 15;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = wn * WTN + j * 32 + 16 * (G & 1) + 4 * (j4 & 3);
            const int c = n >> 3, half = (n >> 2) & 1;
            s16x4 v[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = ks + 8 * (G >> 1) + 4 * h + (j4 >> 2);
                v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(Bs + r * (BN * 2) + swz_b32(r, c) * 16 + half * 8));
            }
            typedef __attribute__((ext_vector_type(8))) short s16x8;
            bfr[j] = __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    auto mma = [&](const bf16x8 (&af)[TM], const bf16x8 (&bfr)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = SWP ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0)
                                : __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    };
    // Fragments of k-slice j are read while the MFMAs of slice j-1 run. The
    // last slice of a stage is multiplied only after the next barrier, so the
    // MFMA pipe still has work while the first reads of the new stage are in
    // flight; its reads must have landed before the barrier (lgkmcnt(0)) since
    // the barrier releases that stage to the next loads.
    constexpr int KS = BK / 16;
    static_assert(KS % 2 == 0, "the deferred slice lives in fragment buffer 1");
    bf16x8 fa[2][TM], fb[2][TN];

    const int nsteps = K / BK;  // >= 2
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < nsteps) issue(s, s * BK);
    for (int s = 0; s < nsteps; ++s) {
        wait_stage<LOADS, NS - 2>(min(NS - 2, nsteps - 1 - s));  // stages after s already issued
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (s + NS - 1 < nsteps) issue((s + NS - 1) % NS, (s + NS - 1) * BK);
        __builtin_amdgcn_sched_barrier(0);
        if (active) {
            lds_u8* As = ring + (s % NS) * STAGE;
            read_frags(As, 0, fa[0], fb[0]);
            if (s > 0) mma(fa[1], fb[1]);
#pragma unroll
            for (int j = 1; j < KS; ++j) {
                read_frags(As, 16 * j, fa[j & 1], fb[j & 1]);
                mma(fa[(j - 1) & 1], fb[(j - 1) & 1]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (!active) return;
    mma(fa[1], fb[1]);
    if constexpr (F8B) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = min(n0 + wn * WTN + j * 32 + (l & 31), N - 1);
            const float sc = bscale[(long)e * N + col];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] *= sc;
        }
    }

    // the epilogue's buffer ranges span this tile's rows only (re - rb can exceed 2^31 bytes of C for one
    // very large group)
    if constexpr (EPI2 != EPI) {
        if (extra) {
            if constexpr (SWP) store_tile32s<TM, TN, WTM, WTN, EPI2>(acc, C, ldc, c_cap, rb, min(re, rb + BM), n0, N, wm, wn);
            else store_tile32<TM, TN, WTM, WTN, EPI2>(acc, C, ldc, c_cap, rb, min(re, rb + BM), n0, N, wm, wn);
            return;
        }
    }
    // the staged epilogues: fp32 row-major, SiLU + bf16 k-blocked, block-scaled fp16
    if constexpr (SWP && WTN == 128 && NS * STAGE >= NW * 16384 && (EPI == 1 || EPI == 0 || EPI == 4)) {
        if ((EPI == 1 && c_cap == 0) || (EPI == 0 && c_cap > 0) || EPI == 4) {
            // every wave's main-loop LDS reads are done before any wave overwrites the ring
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_s_barrier();
            store_tile32s_lds<TM, TN, WTM, WTN, EPI>(acc, C, ldc, c_cap, rb, min(re, rb + BM), n0, N, wm, wn,
                                                     ring + uwave * 16384);
            return;
        }
    }
    if constexpr (SWP) store_tile32s<TM, TN, WTM, WTN, EPI>(acc, C, ldc, c_cap, rb, min(re, rb + BM), n0, N, wm, wn);
    else store_tile32<TM, TN, WTM, WTN, EPI>(acc, C, ldc, c_cap, rb, min(re, rb + BM), n0, N, wm, wn);
}

}  // namespace dma
}  // namespace moe
