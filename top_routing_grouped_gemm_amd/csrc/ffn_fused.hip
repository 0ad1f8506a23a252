// Grouped per-expert FFN with the hidden activation kept on chip: one launch
// computes y_perm[r] = silu(x_perm[r] @ W1[e]) @ W2[e] and h never goes to HBM.
//
// Page 3 (m.lsln.cn/news/228042), section "单机MoE执行流水线": kernel fusion
// merges operators that would otherwise be launched apart, so the fused path
// need not write the intermediate activation back to device memory; it only
// covers certain data types and shapes, and the rest falls back to the
// modular path. Here: bf16, F a multiple of 256 up to 768, H a multiple of 256.
//
// Each workgroup (4 waves, 2 x 2) owns a 64-row M-tile of one expert:
//   phase 1, per 256-column chunk of F: acc = x_tile @ W1[e][:, chunk] over H
//            through a 3-stage direct-to-LDS ring (x rows + W1 slab per 32-k
//            stage), then SiLU, bf16, into h[64][F] in LDS (96 KB at F = 768);
//   phase 2, per 256-column chunk of H: acc = h @ W2[e][:, chunk] over F, A
//            fragments read from the LDS h, W2 slabs through the ring, fp32
//            rows stored to y_perm.
// 64 rows is the largest tile whose h fits beside the ring in 160 KB of LDS.
// The price is the weight feed: every 64-row tile streams its expert's whole
// W1 and W2, 4x the bytes per FLOP of the 256-row tiles of the two-launch path.
#include "gemm_dma.hpp"
#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int kFBM = 64, kFBN = 256, kFBK = 32, kFNS = 3, kFWaves = 4, kFMaxF = 768;
constexpr int kFA = kFBM * kFBK * 2;        // x rows of one stage: 4 KiB, 64 B per row
constexpr int kFB = kFBK * kFBN * 2;        // weight slab of one stage: 16 KiB
constexpr int kFStage = kFA + kFB;
constexpr int kFRing = kFNS * kFStage;      // 60 KiB
constexpr int kFH = kFBM * kFMaxF * 2;      // 96 KiB
static_assert(kFRing + kFH <= 160 * 1024, "LDS");
constexpr int kFAChunks = kFA / (1024 * kFWaves), kFBChunks = kFB / (1024 * kFWaves);  // 1 and 4 per wave

// h[r][*] as 16-byte chunks, chunk c of row r at c ^ (r & 15): the 16 rows one
// 16-lane phase of an A-fragment read touches land in 16 different chunk slots.
__device__ __forceinline__ int swz_h(int r, int c) { return c ^ (r & 15); }

__global__ __launch_bounds__(kFWaves * 64, 1) void ffn_fused_kernel(const uint16_t* __restrict__ xp,
                                                                    const int32_t* __restrict__ offsets, int E,
                                                                    const uint16_t* __restrict__ W1,
                                                                    const uint16_t* __restrict__ W2, int H, int F,
                                                                    float* __restrict__ y) {
    using namespace dma;
    __shared__ __align__(1024) uint8_t smem[kFRing + kFH];
    int e, rb, re, nt;
    if (!xcd_tile<kFBM>(offsets, E, 0, 1, 0, 0x7fffffff, e, rb, re, nt)) return;
    const int wave = threadIdx.x / kWave, l = lane_id();
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const int wm = uwave / 2, wn = uwave % 2;  // 32 rows x 128 columns per wave
    const bool active = rb + wm * 32 < re;     // a wave whose rows all lie past the group skips reads and MFMAs
    lds_u8* ring = (lds_u8*)smem;
    lds_u8* hs = ring + kFRing;
    const uint16_t* W1e = W1 + (long)e * H * F;
    const uint16_t* W2e = W2 + (long)e * F * H;

    // x rows of the tile: lane l fills row 16*uwave + l/4, 16-byte piece l%4 (XOR-swizzled like the GEMM's A)
    const int arow = uwave * 16 + l / 4;
    const uint16_t* a_src = xp + (long)min(rb + arow, re - 1) * H + swz_a32<kFBK>(arow, l % 4) * 8;

    f32x16 acc[1][4];
    auto zero = [&]() {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[0][j][q] = 0.f;
    };
    // B fragments of k-slice ks (16 values) from the stage's [32][256] weight slab (transpose reads)
    auto read_b = [&](lds_u8* Bs, int ks, bf16x8 (&bfr)[4]) {
        const int G = l >> 4, j4 = l & 15;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = wn * 128 + j * 32 + 16 * (G & 1) + 4 * (j4 & 3);
            const int c = n >> 3, half = (n >> 2) & 1;
            s16x4 v[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int r = ks + 8 * (G >> 1) + 4 * hh + (j4 >> 2);
                v[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(Bs + r * (kFBN * 2) + swz_b32(r, c) * 16 + half * 8));
            }
            typedef __attribute__((ext_vector_type(8))) short s16x8;
            bfr[j] = __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    auto mma = [&](const bf16x8& af, const bf16x8 (&bfr)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[0][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr[j], acc[0][j], 0, 0, 0);
    };
    // One GEMM over nsteps k-stages: issue(stage, k0) fills a stage, compute(stage base, step) uses it.
    auto run_ring = [&](int nsteps, auto issue, auto compute, auto waitN) {
#pragma unroll
        for (int s = 0; s < kFNS - 1; ++s)
            if (s < nsteps) issue(s, s * kFBK);
        for (int s = 0; s < nsteps; ++s) {
            waitN(min(kFNS - 2, nsteps - 1 - s));
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (s + kFNS - 1 < nsteps) issue((s + kFNS - 1) % kFNS, (s + kFNS - 1) * kFBK);
            __builtin_amdgcn_sched_barrier(0);
            if (active) compute(ring + (s % kFNS) * kFStage, s);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(VmLgkmWait<0>::value);
        __syncthreads();  // the ring is free for the next GEMM
    };

    // ---- phase 1: h = silu(x_tile @ W1[e]) into LDS, 256 columns of F at a time
    for (int n0 = 0; n0 < F; n0 += kFBN) {
        const uint16_t* b_src[kFBChunks];
#pragma unroll
        for (int i = 0; i < kFBChunks; ++i) {
            const int c = uwave + kFWaves * i;
            const int row = c * 2 + l / 32;
            b_src[i] = W1e + (long)row * F + n0 + swz_b32(row, l % 32) * 8;
        }
        auto issue = [&](int stage, int k0) {
            const uint32_t b0 = (uint32_t)(uintptr_t)(ring + stage * kFStage) + uwave * 1024;
            lds_dma16(a_src + k0, b0);
#pragma unroll
            for (int i = 0; i < kFBChunks; ++i) lds_dma16(b_src[i] + (long)k0 * F, b0 + kFA + i * 1024 * kFWaves);
        };
        auto compute = [&](lds_u8* As, int) {
#pragma unroll
            for (int ks = 0; ks < kFBK; ks += 16) {
                const int row = wm * 32 + (l & 31);
                const bf16x8 af = *(lds_bf16x8*)(As + row * (kFBK * 2) + swz_a32<kFBK>(row, (ks >> 3) + (l >> 5)) * 16);
                bf16x8 bfr[4];
                read_b(As + kFA, ks, bfr);
                mma(af, bfr);
            }
        };
        zero();
        run_ring(H / kFBK, issue, compute, [](int a) { wait_stage<kFAChunks + kFBChunks, kFNS - 2>(a); });
        if (active) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    float v[4] = {acc[0][j][4 * p], acc[0][j][4 * p + 1], acc[0][j][4 * p + 2], acc[0][j][4 * p + 3]};
                    quad_transpose(v);
                    const int row = wm * 32 + 8 * p + 4 * (l >> 5) + (l & 3);
                    const int col = n0 + wn * 128 + j * 32 + ((l & 31) & ~3);
                    const u32x2 pk = {pack_bf16x2(silu_f32(v[0]), silu_f32(v[1])),
                                      pack_bf16x2(silu_f32(v[2]), silu_f32(v[3]))};
                    *(__attribute__((address_space(3))) u32x2*)(hs + row * (F * 2) + swz_h(row, col >> 3) * 16 +
                                                                (col & 7) * 2) = pk;
                }
        }
    }
    __syncthreads();  // h complete

    // ---- phase 2: y_perm rows = h @ W2[e], 256 columns of H at a time
    for (int n0 = 0; n0 < H; n0 += kFBN) {
        const uint16_t* b_src[kFBChunks];
#pragma unroll
        for (int i = 0; i < kFBChunks; ++i) {
            const int c = uwave + kFWaves * i;
            const int row = c * 2 + l / 32;
            b_src[i] = W2e + (long)row * H + n0 + swz_b32(row, l % 32) * 8;
        }
        auto issue = [&](int stage, int k0) {
            const uint32_t b0 = (uint32_t)(uintptr_t)(ring + stage * kFStage) + kFA + uwave * 1024;
#pragma unroll
            for (int i = 0; i < kFBChunks; ++i) lds_dma16(b_src[i] + (long)k0 * H, b0 + i * 1024 * kFWaves);
        };
        auto compute = [&](lds_u8* As, int s) {
#pragma unroll
            for (int ks = 0; ks < kFBK; ks += 16) {
                const int row = wm * 32 + (l & 31);
                const int chunk = (s * kFBK + ks) / 8 + (l >> 5);
                const bf16x8 af = *(lds_bf16x8*)(hs + row * (F * 2) + swz_h(row, chunk) * 16);
                bf16x8 bfr[4];
                read_b(As + kFA, ks, bfr);
                mma(af, bfr);
            }
        };
        zero();
        run_ring(F / kFBK, issue, compute, [](int a) { wait_stage<kFBChunks, kFNS - 2>(a); });
        if (active) store_tile32<1, 4, 32, 128, 1>(acc, y, H, 0, rb, min(re, rb + kFBM), n0, H, wm, wn);
    }
}

}  // namespace

bool ffn_fused_ok(int H, int F, Dtype dt) {
    return dt == kBF16 && F % kFBN == 0 && F <= kFMaxF && H % kFBN == 0;
}

hipError_t launch_ffn_fused(const void* x_perm, const int32_t* offsets, int E, int max_rows, const void* W1,
                            const void* W2, int H, int F, float* y_perm, hipStream_t s) {
    const long grid = (long)(max_rows + kFBM - 1) / kFBM + (E < max_rows ? E : max_rows) + dma::kXcds;
    if (max_rows == 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(ffn_fused_kernel, dim3((unsigned)grid), dim3(kFWaves * 64), 0, s, (const uint16_t*)x_perm,
                       offsets, E, (const uint16_t*)W1, (const uint16_t*)W2, H, F, y_perm);
    return hipGetLastError();
}

}  // namespace moe
