// Grouped per-expert FFN: two ragged GEMM launches over all experts at once.
//
// Page 1 ("MoE大模型的智能调度…", www.jsqmd.com/news/1091713), section 2.2,
// expert layer: each expert is its own two-layer FFN (W1, W2). Page 3
// (m.lsln.cn/news/228042), section "单机MoE执行流水线": one grouped-GEMM
// launch runs every expert matrix although their row counts differ, then the
// experts apply the activation and the output projection; section
// "一个批次如何变成各专家专属的矩阵": decode gives experts one or two rows,
// prefill many.
//
//   up:   h[r]      = silu(x_perm[r] @ W1[e])   (SiLU fused in the epilogue)
//   down: y_perm[r] = h[r] @ W2[e]              (fp32 out, or block-scaled fp16)
//
// Scheduling: the M-tiles of all experts form one ragged sequence (expert e
// contributes ceil(count_e / BM) tiles); each workgroup takes one (M-tile,
// N-tile) pair and finds its expert with a wave-parallel prefix sum over the
// device-side offsets, so no row count ever travels to the host. The grid is
// sized for the worst case (ceil(rows/BM) + min(E, rows) M-tiles) and
// workgroups past the last tile exit at once.
//
// bf16 shapes the direct-to-LDS pipeline of gemm_dma.hpp takes (K a multiple
// of its k-stage, 16-byte rows) run there, in a shape chosen from the mean
// rows per expert (choose_tile): 256x256 tiles for >= 96, 32-row weight-
// streaming tiles for < 24, both over disjoint groups in between. Other bf16
// shapes run the register-staged kernel below (256 threads, BM x BN x 64 tiles
// staged in LDS with one prefetched stage in flight, 16x16x32 bf16 MFMA, fp32
// accumulation); fp32 inputs run the plain-FMA kernel. The fp8-weight (F8B)
// and MX fp8 variants use the same schedule on the shapes further down.
#include <math.h>

#include <limits.h>

#include "gemm_dma.hpp"
#include "gemm_mx.hpp"
#include "mfma_tiles.hpp"
#include "moe_internal.hpp"

namespace moe {

namespace {

// Expert and row range of ragged M-tile `mt`. Returns false past the last tile.
template <int BM>
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int mt, int& e_out,
                                          int& rb, int& re) {
    const int l = lane_id();
    const int per = (E + kWave - 1) / kWave;
    const int e0 = l * per, e1 = min(E, e0 + per);
    int s = 0;
    for (int e = e0; e < e1; ++e) {
        const int c = offsets[e + 1] - offsets[e];
        s += (c + BM - 1) / BM;
    }
    const int incl = wave_incl_scan(s);
    const unsigned long long own = __ballot(mt < incl);
    if (own == 0ull) return false;
    const int L = __ffsll((long long)own) - 1;
    int before = __shfl(incl - s, L, kWave);
    const int eL0 = L * per, eL1 = min(E, eL0 + per);
    int e = eL0;
    for (; e < eL1; ++e) {
        const int c = offsets[e + 1] - offsets[e];
        const int tt = (c + BM - 1) / BM;
        if (mt < before + tt) break;
        before += tt;
    }
    e_out = e;
    rb = offsets[e] + (mt - before) * BM;
    re = offsets[e + 1];
    return true;
}

template <int BM>
__device__ __forceinline__ bool locate(const int32_t* __restrict__ offsets, int E, int fixed_rows, int mt, int& e,
                                       int& rb, int& re) {
    if (offsets == nullptr) {
        e = 0;
        rb = mt * BM;
        re = fixed_rows;
        return rb < re;
    }
    return find_tile<BM>(offsets, E, mt, e, rb, re);
}

enum { kEpiSiluOut = 0, kEpiF32Out = 1, kEpiScaled16 = 4 };

template <int BM, int BN, int BK, int WM, int WN, int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ A, long lda, const uint16_t* __restrict__ B, long strideB, long ldb,
    void* __restrict__ C, long ldc, const int32_t* __restrict__ offsets, int E, int fixed_rows, int N, int K,
    int n_tiles) {
    constexpr int S = BK + 8;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    static_assert(WM * WN == 4, "4 waves");
    static_assert(TM >= 1 && TN >= 1 && BK % 32 == 0, "tile shape");
    constexpr int APT = (BM * BK / 8 + 255) / 256;
    __shared__ __align__(16) uint16_t As[BM * S];
    __shared__ __align__(16) uint16_t Bs[BN * S];

    const int nt = blockIdx.x % n_tiles;
    const int mt = blockIdx.x / n_tiles;
    int e, rb, re;
    if (!locate<BM>(offsets, E, fixed_rows, mt, e, rb, re)) return;
    re = min(re, rb + BM);
    const uint16_t* Be = B + (long)e * strideB;
    const int n0 = nt * BN;

    const int wave = threadIdx.x / kWave, l = lane_id();
    const int wm = wave / WN, wn = wave % WN;

    u32x4 areg[APT];
    BTile<BK, BN, 256> breg;
    load_a_tile_regs<BM, BK, 256>(A, lda, rb, re, K, 0, areg);
    breg.load(Be, ldb, K, N, 0, n0);
    store_a_tile_lds<BM, BK, 256, S>(As, areg);
    breg.template store<S>(Bs);
    __syncthreads();

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < K; k0 += BK) {
        const bool more = k0 + BK < K;
        if (more) {
            load_a_tile_regs<BM, BK, 256>(A, lda, rb, re, K, k0 + BK, areg);
            breg.load(Be, ldb, K, N, k0 + BK, n0);
        }
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *(const bf16x8*)(As + (wm * WTM + i * 16 + (l & 15)) * S + kk + (l >> 4) * 8);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bfr[j] = *(const bf16x8*)(Bs + (wn * WTN + j * 16 + (l & 15)) * S + kk + (l >> 4) * 8);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
        if (more) {
            store_a_tile_lds<BM, BK, 256, S>(As, areg);
            breg.template store<S>(Bs);
            __syncthreads();
        }
    }

#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * WTN + j * 16 + (l & 15);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = rb + wm * WTM + i * 16 + (l >> 4) * 4 + q;
                if (row < re && col < N) {
                    const float v = acc[i][j][q];
                    if (EPI == kEpiSiluOut)
                        ((uint16_t*)C)[(long)row * ldc + col] = (uint16_t)f32_to_bf16_bits(silu_f32(v));
                    else
                        ((float*)C)[(long)row * ldc + col] = v;
                }
            }
        }
}

// fp32 path: 32x32 tiles on plain FMA, 2x2 outputs per thread.
template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(const float* __restrict__ A, long lda,
                                                               const float* __restrict__ B, long strideB, long ldb,
                                                               void* __restrict__ C, long ldc,
                                                               const int32_t* __restrict__ offsets, int E,
                                                               int fixed_rows, int N, int K, int n_tiles) {
    constexpr int BM = 32, BN = 32, BK = 16;
    __shared__ float As[BK][BM + 1];
    __shared__ float Bs[BK][BN + 1];
    const int nt = blockIdx.x % n_tiles;
    const int mt = blockIdx.x / n_tiles;
    int e, rb, re;
    if (!locate<BM>(offsets, E, fixed_rows, mt, e, rb, re)) return;
    re = min(re, rb + BM);
    const float* Be = B + (long)e * strideB;
    const int n0 = nt * BN;
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    for (int k0 = 0; k0 < K; k0 += BK) {
        for (int i = threadIdx.x; i < BK * BM; i += 256) {
            const int m = i / BK, kk = i % BK;
            const int r = rb + m, kg = k0 + kk;
            As[kk][m] = (r < re && kg < K) ? A[(long)r * lda + kg] : 0.0f;
        }
        for (int i = threadIdx.x; i < BK * BN; i += 256) {
            const int kk = i / BN, n = i % BN;
            const int kg = k0 + kk, ng = n0 + n;
            Bs[kk][n] = (kg < K && ng < N) ? Be[(long)kg * ldb + ng] : 0.0f;
        }
        __syncthreads();
        for (int kk = 0; kk < BK; ++kk) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[a][b] = fmaf(As[kk][ty * 2 + a], Bs[kk][tx * 2 + b], acc[a][b]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int row = rb + ty * 2 + a, col = n0 + tx * 2 + b;
            if (row < re && col < N) {
                float v = acc[a][b];
                if (EPI == kEpiSiluOut) v = v / (1.0f + expf(-v));
                ((float*)C)[(long)row * ldc + col] = v;
            }
        }
}

inline long max_mtiles(int bm, const int32_t* offsets, int E, int fixed_rows, int max_rows) {
    if (offsets == nullptr) return (fixed_rows + bm - 1) / bm;
    long groups = E < max_rows ? E : max_rows;
    return (max_rows + bm - 1) / bm + groups;
}

template <int BM, int BN, int BK, int WM, int WN, int EPI>
hipError_t run_bf16(const void* A, long lda, const void* B, long strideB, long ldb, void* C, long ldc,
                    const int32_t* offsets, int E, int fixed_rows, int max_rows, int N, int K, hipStream_t s) {
    const int n_tiles = (N + BN - 1) / BN;
    const long grid = max_mtiles(BM, offsets, E, fixed_rows, max_rows) * n_tiles;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<BM, BN, BK, WM, WN, EPI>), dim3((unsigned)grid), dim3(256), 0, s,
                       (const uint16_t*)A, lda, (const uint16_t*)B, strideB, ldb, C, ldc, offsets, E, fixed_rows, N,
                       K, n_tiles);
    return hipGetLastError();
}

// Direct-to-LDS pipelines (gemm_dma.hpp), one shape per regime:
//  - DmaLarge: many rows per group (prefill). 256x256 tiles, 32-wide
//    k-stages, a 4-stage ring, 8 waves; MFMA-bound when fed.
//  - DmaStream: a few rows per group (decode). Each tile is one 32-row MFMA
//    block against a 128-column weight slab; 64-wide k-stages in a 4-stage
//    ring (80 KB) let two workgroups share a CU, so ~120 KB of weight loads
//    stay in flight per CU and one workgroup's pipeline fill overlaps the
//    other's tail (measured: 6 stages with one workgroup per CU streamed
//    4.7 TB/s, 4 stages with two 5.5 TB/s; with non-temporal weight loads
//    6.1-6.2 TB/s).
template <int BM_, int BN_, int BK_, int NS_, int WM_, int WN_>
struct DmaCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, NS = NS_, WM = WM_, WN = WN_;
};
using DmaLarge = DmaCfg<256, 256, 32, 4, 4, 2>;
using DmaStream = DmaCfg<32, 128, 64, 4, 1, 4>;

// a_kstep / c_cap: see gemm32_kernel (1 / 0 for row-major A / C).
// [rmin, rmax): the group sizes this launch takes (see xcd_tile).
// xg: one more group after the E groups (the shared expert), stored with EPI2.
template <class C, int EPI, int EPI2 = EPI>
hipError_t run_dma(const void* A, long lda, long a_kstep, const int32_t* a_rows, const void* B, long strideB, long ldb,
                   void* Cm, long ldc, long c_cap, const int32_t* offsets, int E, int fixed_rows, int max_rows, int N,
                   int K, hipStream_t s, int rmin = 0, int rmax = INT_MAX, dma::ExtraGroup xg = dma::ExtraGroup{}) {
    const int n_tiles = (N + C::BN - 1) / C::BN;
    if (xg.rows > 0 && offsets == nullptr) return hipErrorInvalidValue;
    // XCD-chunked order needs up to kXcds-1 spare workgroups past the tile count
    const long grid =
        (max_mtiles(C::BM, offsets, E, fixed_rows, max_rows) + (xg.rows + C::BM - 1) / C::BM) * n_tiles + dma::kXcds;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((dma::gemm32_kernel<C::BM, C::BN, C::BK, C::NS, C::WM, C::WN, EPI, false, EPI2>),
                       dim3((unsigned)grid), dim3(C::WM * C::WN * 64), 0, s, (const uint16_t*)A, lda, a_kstep, a_rows,
                       B, strideB, ldb, nullptr, Cm, ldc, c_cap, offsets, E, fixed_rows, rmin, rmax, N, K, n_tiles,
                       xg);
    return hipGetLastError();
}

// fp8-weight shapes (gemm32_kernel with F8B): a B stage is whole 128 x 64
// code tiles, so BK is 64 and the byte count per stage halves. The streaming
// shape runs 3-stage rings of 36 KB, four workgroups per CU (measured at
// decode: 3 stages x 4 workgroups streamed 4.7-4.8 TB/s of weights, 4 x 3
// 4.6, 6 x 2 4.1, 8 x 1 3.5); the large shape's 64-wide k-stages also give A
// 128-byte row pieces.
using F8Stream = DmaCfg<32, 128, 64, 3, 1, 4>;
using F8Large = DmaCfg<256, 256, 64, 3, 4, 2>;

template <class C, int EPI>
hipError_t run_dma8(const void* A, long lda, const int32_t* a_rows, const void* Bq, long strideB, const float* bscale,
                    void* Cm, long ldc, long c_cap, const int32_t* offsets, int E, int max_rows, int N, int K,
                    hipStream_t s, int rmin = 0, int rmax = INT_MAX) {
    const int n_tiles = (N + C::BN - 1) / C::BN;
    const long grid = max_mtiles(C::BM, offsets, E, 0, max_rows) * n_tiles + dma::kXcds;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((dma::gemm32_kernel<C::BM, C::BN, C::BK, C::NS, C::WM, C::WN, EPI, true>),
                       dim3((unsigned)grid), dim3(C::WM * C::WN * 64), 0, s, (const uint16_t*)A, lda, 1L, a_rows, Bq,
                       strideB, 0L, bscale, Cm, ldc, c_cap, offsets, E, 0, rmin, rmax, N, K, n_tiles,
                       dma::ExtraGroup{});
    return hipGetLastError();
}

// The three row regimes of choose_tile on the fp8 shapes.
template <int EPI>
hipError_t run_fp8_cfg(TileCfg cfg, const void* A, long lda, const int32_t* a_rows, const void* Bq, long strideB,
                       const float* bscale, void* Cm, long ldc, long c_cap, const int32_t* offsets, int E,
                       int max_rows, int N, int K, hipStream_t s) {
    if (cfg == kTileM128)
        return run_dma8<F8Large, EPI>(A, lda, a_rows, Bq, strideB, bscale, Cm, ldc, c_cap, offsets, E, max_rows, N, K,
                                      s);
    if (cfg == kTileMixed) {
        const hipError_t e = run_dma8<F8Stream, EPI>(A, lda, a_rows, Bq, strideB, bscale, Cm, ldc, c_cap, offsets, E,
                                                     max_rows, N, K, s, 0, kStreamRows);
        if (e != hipSuccess) return e;
        return run_dma8<F8Large, EPI>(A, lda, a_rows, Bq, strideB, bscale, Cm, ldc, c_cap, offsets, E, max_rows, N, K,
                                      s, kStreamRows, INT_MAX);
    }
    return run_dma8<F8Stream, EPI>(A, lda, a_rows, Bq, strideB, bscale, Cm, ldc, c_cap, offsets, E, max_rows, N, K,
                                   s);
}

// MX fp8 shape (gemm_mx_kernel): 256 x 256 tiles, 64-k stages of 34 KB
// (codes of A and B plus their scale dwords), a 4-stage ring, 8 waves.
struct MxLarge {
    static constexpr int BM = 256, BN = 256, NS = 4, WM = 4, WN = 2;
};

// Weight-streaming MX shape (dma::gemm_mx_stream_kernel): 32 x 128 tiles,
// 128-k stages of 21 KB in a 3-stage ring, two workgroups per CU.
constexpr int kMxStreamNS = 3;

template <class C, int EPI>
hipError_t run_mx(const void* A, long a_kstride, long a_rstride, const int32_t* a_rows, const void* a_sc,
                  long a_sc_rows, const void* B, long strideB, const void* b_sc, long b_sc_estride, int Npad,
                  void* Cm, long ldc, long c_cap, void* c_sc, const int32_t* offsets, int E, int max_rows, int N,
                  int K, hipStream_t s, int rmin = 0, int rmax = INT_MAX) {
    const int n_tiles = (N + C::BN - 1) / C::BN;
    const long grid = max_mtiles(C::BM, offsets, E, 0, max_rows) * n_tiles + dma::kXcds;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((dma::gemm_mx_kernel<C::BM, C::BN, C::NS, C::WM, C::WN, EPI>), dim3((unsigned)grid),
                       dim3(C::WM * C::WN * 64), 0, s, (const uint8_t*)A, a_kstride, a_rstride, a_rows,
                       (const uint8_t*)a_sc, a_sc_rows, (const uint8_t*)B, strideB, (const uint8_t*)b_sc,
                       b_sc_estride, Npad, Cm, ldc, c_cap, (uint8_t*)c_sc, offsets, E, rmin, rmax, N, K, n_tiles);
    return hipGetLastError();
}

template <int EPI>
hipError_t run_mx_stream(const void* A, long a_kstride, long a_rstride, const int32_t* a_rows, const void* a_sc,
                         long a_sc_rows, const void* B, long strideB, const void* b_sc, long b_sc_estride, int Npad,
                         void* Cm, long ldc, long c_cap, void* c_sc, const int32_t* offsets, int E, int max_rows,
                         int N, int K, hipStream_t s, int rmin = 0, int rmax = INT_MAX) {
    const int n_tiles = (N + dma::kMxTileN - 1) / dma::kMxTileN;
    const long grid = max_mtiles(32, offsets, E, 0, max_rows) * n_tiles + dma::kXcds;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((dma::gemm_mx_stream_kernel<kMxStreamNS, EPI>), dim3((unsigned)grid), dim3(256), 0, s,
                       (const uint8_t*)A, a_kstride, a_rstride, a_rows, (const uint8_t*)a_sc, a_sc_rows,
                       (const uint8_t*)B, strideB, (const uint8_t*)b_sc, b_sc_estride, Npad, Cm, ldc, c_cap,
                       (uint8_t*)c_sc, offsets, E, rmin, rmax, N, K, n_tiles);
    return hipGetLastError();
}

// The MX products over all groups in the regimes of choose_tile: 256-row
// tiles, 32-row weight-streaming tiles, or both over disjoint groups.
template <int EPI>
hipError_t run_mx_cfg(const void* A, long a_kstride, long a_rstride, const int32_t* a_rows, const void* a_sc,
                      long a_sc_rows, const void* B, long strideB, const void* b_sc, long b_sc_estride, int Npad,
                      void* Cm, long ldc, long c_cap, void* c_sc, const int32_t* offsets, int E, int max_rows, int N,
                      int K, hipStream_t s) {
    const TileCfg cfg = choose_tile(max_rows, E);
    if (cfg == kTileM128)
        return run_mx<MxLarge, EPI>(A, a_kstride, a_rstride, a_rows, a_sc, a_sc_rows, B, strideB, b_sc, b_sc_estride,
                                    Npad, Cm, ldc, c_cap, c_sc, offsets, E, max_rows, N, K, s);
    const int split = cfg == kTileMixed ? kStreamRows : INT_MAX;
    const hipError_t e = run_mx_stream<EPI>(A, a_kstride, a_rstride, a_rows, a_sc, a_sc_rows, B, strideB, b_sc,
                                            b_sc_estride, Npad, Cm, ldc, c_cap, c_sc, offsets, E, max_rows, N, K, s,
                                            0, split);
    if (e != hipSuccess || cfg != kTileMixed) return e;
    return run_mx<MxLarge, EPI>(A, a_kstride, a_rstride, a_rows, a_sc, a_sc_rows, B, strideB, b_sc, b_sc_estride,
                                Npad, Cm, ldc, c_cap, c_sc, offsets, E, max_rows, N, K, s, split, INT_MAX);
}

template <class C>
bool dma_ok(long lda, long ldb, int N, int K) {
    return K % C::BK == 0 && K >= 2 * C::BK && N % 8 == 0 && N >= 8 && lda % 8 == 0 && ldb % 8 == 0;
}

// h_cap > 0: the k-blocked h layout (W1 writes it as C, W2 reads it as A);
// only the large direct-to-LDS shape takes it (h_blocked decides).
// xg (large-tile shape only, see ffn_shared_merges): the shared expert's group.
template <int EPI>
hipError_t run_bf16_cfg(TileCfg cfg, const void* A, long lda, const void* B, long strideB, long ldb, void* C,
                        long ldc, const int32_t* offsets, int E, int fixed_rows, int max_rows, int N, int K,
                        long h_cap, hipStream_t s, dma::ExtraGroup xg = dma::ExtraGroup{}) {
    if (h_cap > 0) {
        if (EPI == kEpiSiluOut)  // W1: C = h blocked
            return run_dma<DmaLarge, EPI>(A, lda, 1, nullptr, B, strideB, ldb, C, ldc, h_cap, offsets, E, fixed_rows,
                                          max_rows, N, K, s, 0, INT_MAX, xg);
        return run_dma<DmaLarge, EPI>(A, 32, h_cap, nullptr, B, strideB, ldb, C, ldc, 0, offsets, E, fixed_rows,
                                      max_rows, N, K, s, 0, INT_MAX, xg);  // W2: A = h blocked
    }
    if (xg.rows > 0 && (cfg != kTileM128 || !dma_ok<DmaLarge>(lda, ldb, N, K))) return hipErrorInvalidValue;
    switch (cfg) {
        case kTileM128:
            if (dma_ok<DmaLarge>(lda, ldb, N, K))
                return run_dma<DmaLarge, EPI>(A, lda, 1, nullptr, B, strideB, ldb, C, ldc, 0, offsets, E, fixed_rows,
                                              max_rows, N, K, s, 0, INT_MAX, xg);
            return run_bf16<128, 128, 64, 2, 2, EPI>(A, lda, B, strideB, ldb, C, ldc, offsets, E, fixed_rows,
                                                     max_rows, N, K, s);
        case kTileMixed:
            if (offsets != nullptr && dma_ok<DmaStream>(lda, ldb, N, K) && dma_ok<DmaLarge>(lda, ldb, N, K)) {
                const hipError_t e = run_dma<DmaStream, EPI>(A, lda, 1, nullptr, B, strideB, ldb, C, ldc, 0, offsets,
                                                             E, fixed_rows, max_rows, N, K, s, 0, kStreamRows);
                if (e != hipSuccess) return e;
                return run_dma<DmaLarge, EPI>(A, lda, 1, nullptr, B, strideB, ldb, C, ldc, 0, offsets, E, fixed_rows,
                                              max_rows, N, K, s, kStreamRows, INT_MAX);
            }
            return run_bf16<64, 128, 64, 2, 2, EPI>(A, lda, B, strideB, ldb, C, ldc, offsets, E, fixed_rows,
                                                    max_rows, N, K, s);
        case kTileM64:
            return run_bf16<64, 128, 64, 2, 2, EPI>(A, lda, B, strideB, ldb, C, ldc, offsets, E, fixed_rows,
                                                    max_rows, N, K, s);
        default:
            if (dma_ok<DmaStream>(lda, ldb, N, K))
                return run_dma<DmaStream, EPI>(A, lda, 1, nullptr, B, strideB, ldb, C, ldc, 0, offsets, E, fixed_rows,
                                               max_rows, N, K, s);
            return run_bf16<16, 128, 64, 1, 4, EPI>(A, lda, B, strideB, ldb, C, ldc, offsets, E, fixed_rows,
                                                    max_rows, N, K, s);
    }
}

template <int EPI>
hipError_t run_f32(const void* A, long lda, const void* B, long strideB, long ldb, void* C, long ldc,
                   const int32_t* offsets, int E, int fixed_rows, int max_rows, int N, int K, hipStream_t s) {
    const int n_tiles = (N + 31) / 32;
    const long grid = max_mtiles(32, offsets, E, fixed_rows, max_rows) * n_tiles;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((grouped_gemm_f32_kernel<EPI>), dim3((unsigned)grid), dim3(256), 0, s, (const float*)A, lda,
                       (const float*)B, strideB, ldb, C, ldc, offsets, E, fixed_rows, N, K, n_tiles);
    return hipGetLastError();
}

}  // namespace

bool ffn_up_gathers(TileCfg cfg, int H, int F, Dtype dt) {
    if (dt != kBF16) return false;
    if (cfg == kTileM128) return dma_ok<DmaLarge>(H, F, F, H);
    if (cfg == kTileM16) return dma_ok<DmaStream>(H, F, F, H);
    if (cfg == kTileMixed) return dma_ok<DmaLarge>(H, F, F, H) && dma_ok<DmaStream>(H, F, F, H);
    return false;
}

bool ffn_shared_merges(TileCfg cfg, int H, int F, int Fs, Dtype dt) {
    return dt == kBF16 && Fs == F && cfg == kTileM128 && dma_ok<DmaLarge>(H, F, F, H) && dma_ok<DmaLarge>(F, H, H, F);
}

namespace {
// The shared expert as the W1 / W2 launch's extra group (row-major x; its h
// k-blocked when sh.h_cap > 0, like the routed h).
dma::ExtraGroup shared_up(const SharedGroup* sh, int H, int F) {
    if (sh == nullptr) return dma::ExtraGroup{};
    return dma::ExtraGroup{(const uint16_t*)sh->x, H, 1, sh->W1s, sh->h, F, sh->h_cap, sh->T};
}
dma::ExtraGroup shared_down(const SharedGroup* sh, int F, int H) {
    if (sh == nullptr) return dma::ExtraGroup{};
    const bool blk = sh->h_cap > 0;
    return dma::ExtraGroup{(const uint16_t*)sh->h, blk ? 32L : (long)F, blk ? sh->h_cap : 1L, sh->W2s, sh->y, H, 0,
                           sh->T};
}
}  // namespace

hipError_t launch_ffn_up_gather(const void* x, const int32_t* row_token, const int32_t* offsets, int E, int max_rows,
                                const void* W1, int H, int F, TileCfg cfg, long h_cap, void* h, hipStream_t s,
                                const SharedGroup* sh) {
    if (sh != nullptr && cfg != kTileM128) return hipErrorInvalidValue;
    if (cfg == kTileM128)
        return run_dma<DmaLarge, kEpiSiluOut>(x, H, 1, row_token, W1, (long)H * F, F, h, F, h_cap, offsets, E, 0,
                                              max_rows, F, H, s, 0, INT_MAX, shared_up(sh, H, F));
    if (cfg == kTileMixed) {
        const hipError_t e = run_dma<DmaStream, kEpiSiluOut>(x, H, 1, row_token, W1, (long)H * F, F, h, F, 0, offsets,
                                                             E, 0, max_rows, F, H, s, 0, kStreamRows);
        if (e != hipSuccess) return e;
        return run_dma<DmaLarge, kEpiSiluOut>(x, H, 1, row_token, W1, (long)H * F, F, h, F, 0, offsets, E, 0,
                                              max_rows, F, H, s, kStreamRows, INT_MAX);
    }
    return run_dma<DmaStream, kEpiSiluOut>(x, H, 1, row_token, W1, (long)H * F, F, h, F, 0, offsets, E, 0, max_rows,
                                           F, H, s);
}

long h_blocked(TileCfg cfg, int H, int F, long cap, Dtype dt) {
    if (dt != kBF16 || cfg != kTileM128 || F % 32 != 0) return 0;
    if (!dma_ok<DmaLarge>(H, F, F, H) || !dma_ok<DmaLarge>(F, H, H, F)) return 0;
    if (cap * F * 2 > 0x7fff0000L) return 0;  // 32-bit buffer offsets
    return cap;
}

bool ffn_down_packs(TileCfg cfg, int F, int H, Dtype dt) {
    if (dt != kBF16 || H % 32 != 0) return false;  // whole 32-column scale blocks
    if (cfg == kTileM128) return dma_ok<DmaLarge>(F, H, H, F);
    if (cfg == kTileM16) return dma_ok<DmaStream>(F, H, H, F);
    if (cfg == kTileMixed) return dma_ok<DmaLarge>(F, H, H, F) && dma_ok<DmaStream>(F, H, H, F);
    return false;
}

hipError_t launch_ffn_down_packed(const void* h, const int32_t* offsets, int E, int max_rows, const void* W2, int F,
                                  int H, TileCfg cfg, long h_cap, void* y_planes, long cap, hipStream_t s,
                                  const SharedGroup* sh) {
    const long sb = (long)F * H;
    if (sh != nullptr && cfg != kTileM128) return hipErrorInvalidValue;
    if (cfg == kTileM128) {
        // the shared expert's rows go to fp32 y_shared (EPI2), the routed rows to the packed planes
        if (h_cap > 0)
            return run_dma<DmaLarge, kEpiScaled16, kEpiF32Out>(h, 32, h_cap, nullptr, W2, sb, H, y_planes, H, cap,
                                                               offsets, E, 0, max_rows, H, F, s, 0, INT_MAX,
                                                               shared_down(sh, F, H));
        return run_dma<DmaLarge, kEpiScaled16, kEpiF32Out>(h, F, 1, nullptr, W2, sb, H, y_planes, H, cap, offsets, E,
                                                           0, max_rows, H, F, s, 0, INT_MAX, shared_down(sh, F, H));
    }
    if (cfg == kTileMixed) {
        const hipError_t e = run_dma<DmaStream, kEpiScaled16>(h, F, 1, nullptr, W2, sb, H, y_planes, H, cap, offsets,
                                                              E, 0, max_rows, H, F, s, 0, kStreamRows);
        if (e != hipSuccess) return e;
        return run_dma<DmaLarge, kEpiScaled16>(h, F, 1, nullptr, W2, sb, H, y_planes, H, cap, offsets, E, 0, max_rows,
                                               H, F, s, kStreamRows, INT_MAX);
    }
    return run_dma<DmaStream, kEpiScaled16>(h, F, 1, nullptr, W2, sb, H, y_planes, H, cap, offsets, E, 0, max_rows, H,
                                            F, s);
}

bool ffn_fp8_ok(int H, int F) { return H % 64 == 0 && F % 64 == 0 && H >= 128 && F >= 128; }

hipError_t launch_ffn_up_fp8(const void* A, const int32_t* a_rows, const int32_t* offsets, int E, int max_rows,
                             const uint8_t* W1q, const float* s1, int H, int F, TileCfg cfg, void* h, hipStream_t s) {
    const long strideB = fp8_weight_bytes(1, H, F);
    return run_fp8_cfg<kEpiSiluOut>(cfg, A, H, a_rows, W1q, strideB, s1, h, F, 0, offsets, E, max_rows, F, H, s);
}

hipError_t launch_ffn_down_fp8(const void* h, const int32_t* offsets, int E, int max_rows, const uint8_t* W2q,
                               const float* s2, int F, int H, TileCfg cfg, bool packed, void* y, long cap,
                               hipStream_t s) {
    const long strideB = fp8_weight_bytes(1, F, H);
    if (packed)
        return run_fp8_cfg<kEpiScaled16>(cfg, h, F, nullptr, W2q, strideB, s2, y, H, cap, offsets, E, max_rows, H, F,
                                         s);
    return run_fp8_cfg<kEpiF32Out>(cfg, h, F, nullptr, W2q, strideB, s2, y, H, 0, offsets, E, max_rows, H, F, s);
}

bool ffn_mx_ok(int H, int F) { return H % 128 == 0 && F % 128 == 0 && H >= 128 && F >= 128; }

hipError_t launch_ffn_up_mx(const void* xq, const void* xs, long x_rows, const int32_t* row_token,
                            const int32_t* offsets, int E, int max_rows, const uint8_t* W1q, const uint8_t* W1s, int H,
                            int F, void* hq, void* hs, long cap, hipStream_t s) {
    // A: row-major token codes xq[x_rows][H] gathered through row_token, scales [H/128][x_rows][4]
    return run_mx_cfg<3>(xq, dma::kMxBK, H, row_token, xs, x_rows, W1q, mx_weight_bytes(1, H, F), W1s,
                         mx_weight_scale_bytes(1, H, F), F, hq, 0, cap, hs, offsets, E, max_rows, F, H, s);
}

hipError_t launch_ffn_down_mx(const void* hq, const void* hs, long cap, const int32_t* offsets, int E, int max_rows,
                              const uint8_t* W2q, const uint8_t* W2s, int F, int H, bool packed, void* y,
                              hipStream_t s) {
    // A: the k-blocked h codes [F/64][cap][64] of the W1 launch, scales [F/128][cap][4]
    const long ks = cap * dma::kMxBK;
    if (packed)
        return run_mx_cfg<kEpiScaled16>(hq, ks, dma::kMxBK, nullptr, hs, cap, W2q, mx_weight_bytes(1, F, H), W2s,
                                        mx_weight_scale_bytes(1, F, H), H, y, H, cap, nullptr, offsets, E, max_rows,
                                        H, F, s);
    return run_mx_cfg<kEpiF32Out>(hq, ks, dma::kMxBK, nullptr, hs, cap, W2q, mx_weight_bytes(1, F, H), W2s,
                                  mx_weight_scale_bytes(1, F, H), H, y, H, 0, nullptr, offsets, E, max_rows, H, F,
                                  s);
}

TileCfg choose_tile(long rows, int groups) {
    const long mean = groups > 0 ? rows / groups : rows;
    if (mean >= 96) return kTileM128;
    if (mean >= 24) return kTileMixed;
    return kTileM16;
}

hipError_t launch_ffn_up(const void* A, const int32_t* offsets, int E, int fixed_rows, int max_rows, const void* W1,
                         int H, int F, Dtype dt, void* h, TileCfg cfg, long h_cap, hipStream_t s,
                         const SharedGroup* sh) {
    const long strideB = (offsets == nullptr) ? 0 : (long)H * F;
    if (sh != nullptr && (dt != kBF16 || offsets == nullptr)) return hipErrorInvalidValue;
    if (dt == kBF16)
        return run_bf16_cfg<kEpiSiluOut>(cfg, A, H, W1, strideB, F, h, F, offsets, E, fixed_rows, max_rows, F, H,
                                         h_cap, s, shared_up(sh, H, F));
    return run_f32<kEpiSiluOut>(A, H, W1, strideB, F, h, F, offsets, E, fixed_rows, max_rows, F, H, s);
}

hipError_t launch_ffn_down(const void* h, const int32_t* offsets, int E, int fixed_rows, int max_rows,
                           const void* W2, int F, int H, Dtype dt, float* y, TileCfg cfg, long h_cap, hipStream_t s,
                           const SharedGroup* sh) {
    const long strideB = (offsets == nullptr) ? 0 : (long)F * H;
    if (sh != nullptr && (dt != kBF16 || offsets == nullptr)) return hipErrorInvalidValue;
    if (dt == kBF16)
        return run_bf16_cfg<kEpiF32Out>(cfg, h, F, W2, strideB, H, y, H, offsets, E, fixed_rows, max_rows, H, F, h_cap,
                                        s, shared_down(sh, F, H));
    return run_f32<kEpiF32Out>(h, F, W2, strideB, H, y, H, offsets, E, fixed_rows, max_rows, H, F, s);
}

}  // namespace moe
