// Router: logits = x @ Wr + bias, top-k with ties to the lower expert id,
// softmax over the selected logits, optional drop-and-renormalise.
//
// Page 1 ("MoE大模型的智能调度…", www.jsqmd.com/news/1091713), section 2.2,
// routing layer: score the experts, soft top-k (softmax over the kept
// logits), zero any weight under the threshold and renormalise. Page 3
// (m.lsln.cn/news/228042), section "单机MoE执行流水线": the router scores
// every expert and top-k keeps the chosen indices and their weights.
//
// bf16: one workgroup (4 waves) takes 16 or 32 tokens; the logits block is a
// small GEMM on the matrix cores (bf16 products, fp32 accumulation) with Wr
// transposed into LDS. The fp32 logits then go to LDS and each wave runs the
// top-k of one token at a time (a ballot-based radix select); the logits are
// never written to memory.
#include <float.h>
#include <math.h>

#include "gemm_dma.hpp"
#include "mfma_tiles.hpp"
#include "moe_internal.hpp"
#include "topk.hpp"

namespace moe {

namespace {

constexpr int kRouteBK = 32;
constexpr int kRouteS = kRouteBK + 8;  // LDS row stride (bf16 elements)
constexpr int kQMax = 16;              // experts per lane: E <= 1024

// Top-k of one token whose E logits sit in LDS at lg[0..E) (E <= 64*Q), one
// whole wave: radix select, softmax over the selection (+ drop), slots in
// ascending expert id (topk.hpp).
template <int Q, bool EARLY = false>
__device__ void topk_select(const float* lg, int E, int k, float drop, long t, int32_t* __restrict__ ids,
                            float* __restrict__ wout) {
    const int l = lane_id();
    float v[Q];
    uint32_t key[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int e = q * kWave + l;
        v[q] = e < E ? lg[e] : -INFINITY;
        key[q] = e < E ? ord_key(v[q] + 0.0f) : 0u;
    }
    bool sel[Q], kept[Q];
    float p[Q];
    radix_select<Q, EARLY>(key, k, sel);
    softmax_drop<Q>(v, sel, drop, p, kept);
    write_slots<Q>(sel, kept, p, t, k, ids, wout);
}

// For kernels whose E is only known at run time; the kernels templated on the
// padded expert count EP call topk_select<EP/64> directly (measured on the
// prefill router's reduction: 9.2 -> 7.6 us, the top-k part 5.2 -> 3.6 us).
__device__ void topk_one_token(const float* lg, int E, int k, float drop, long t, int32_t* __restrict__ ids,
                               float* __restrict__ wout) {
    if (E <= kWave) topk_select<1>(lg, E, k, drop, t, ids, wout);
    else if (E <= 2 * kWave) topk_select<2>(lg, E, k, drop, t, ids, wout);
    else if (E <= 4 * kWave) topk_select<4>(lg, E, k, drop, t, ids, wout);
    else if (E <= 8 * kWave) topk_select<8>(lg, E, k, drop, t, ids, wout);
    else topk_select<kQMax>(lg, E, k, drop, t, ids, wout);
}

template <int MT, int NTW, bool VEC>
__global__ __launch_bounds__(256) void route_bf16_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ Wr,
                                                         const float* __restrict__ bias, int T, int H, int E,
                                                         int k, float drop, int32_t* __restrict__ ids,
                                                         float* __restrict__ wout) {
    constexpr int RT = MT * 16;
    extern __shared__ __align__(16) uint8_t smem[];
    const int EP = (E + 15) & ~15;
    uint16_t* As = (uint16_t*)smem;
    uint16_t* Bs = As + RT * kRouteS;
    float* lg = (float*)smem;  // reused after the K loop

    const int t0 = blockIdx.x * RT;
    const int wave = threadIdx.x / kWave, l = lane_id();
    const int ntiles = EP / 16;

    f32x4 acc[MT][NTW];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < H; k0 += kRouteBK) {
        // x rows t0 .. t0+RT, k-contiguous
        for (int i = threadIdx.x; i < RT * (kRouteBK / 8); i += 256) {
            const int m = i / (kRouteBK / 8), kv = i % (kRouteBK / 8);
            const int t = t0 + m, kk = k0 + kv * 8;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (t < T && kk < H) v = *(const u32x4*)(x + (long)t * H + kk);
            *(u32x4*)(As + m * kRouteS + kv * 8) = v;
        }
        // Wr rows k0 .. k0+BK, transposed into Bs[e][k]
        if (VEC) {
            for (int i = threadIdx.x; i < (kRouteBK / 4) * (EP / 8); i += 256) {
                const int nv = i % (EP / 8), kb = i / (EP / 8);
                const int n = nv * 8;
                u32x4 r[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int kk = k0 + kb * 4 + q;
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (n < E && kk < H) v = *(const u32x4*)(Wr + (long)kk * E + n);
                    r[q] = v;
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int ws = c >> 1;
                    const bool hi = c & 1;
                    uint32_t e0 = hi ? (r[0][ws] >> 16) : (r[0][ws] & 0xFFFFu);
                    uint32_t e1 = hi ? (r[1][ws] >> 16) : (r[1][ws] & 0xFFFFu);
                    uint32_t e2 = hi ? (r[2][ws] >> 16) : (r[2][ws] & 0xFFFFu);
                    uint32_t e3 = hi ? (r[3][ws] >> 16) : (r[3][ws] & 0xFFFFu);
                    *(u32x2*)(Bs + (n + c) * kRouteS + kb * 4) = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
                }
            }
        } else {
            for (int i = threadIdx.x; i < kRouteBK * EP; i += 256) {
                const int n = i % EP, kr = i / EP;
                const int kk = k0 + kr;
                const uint16_t v = (n < E && kk < H) ? Wr[(long)kk * E + n] : (uint16_t)0;
                Bs[n * kRouteS + kr] = v;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kRouteBK; kk += 32) {
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int nt = wave + 4 * j;
                if (nt < ntiles) {
                    const uint16_t* brow = Bs + (nt * 16 + (l & 15)) * kRouteS + kk + (l >> 4) * 8;
#pragma unroll
                    for (int i = 0; i < MT; ++i) {
                        const uint16_t* arow = As + (i * 16 + (l & 15)) * kRouteS + kk + (l >> 4) * 8;
                        acc[i][j] = mfma_bf16_16x16x32(arow, brow, acc[i][j]);
                    }
                }
            }
        }
        __syncthreads();
    }
    // logits (+ bias) -> LDS [RT][EP]
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int nt = wave + 4 * j;
        if (nt < ntiles) {
            const int e = nt * 16 + (l & 15);
            const float b = (bias != nullptr && e < E) ? bias[e] : 0.0f;
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int m = i * 16 + (l >> 4) * 4 + q;
                    lg[m * EP + e] = acc[i][j][q] + b;
                }
        }
    }
    __syncthreads();
    for (int m = wave; m < RT; m += 4) {
        const long t = t0 + m;
        if (t < T) topk_one_token(lg + m * EP, E, k, drop, t, ids, wout);
    }
}

// fp32 router: plain FMA logits (the fp32 path serves small layers).
constexpr int kRouteF32Rows = 16;
constexpr int kRouteF32Chunk = 64;

__global__ __launch_bounds__(256) void route_f32_kernel(const float* __restrict__ x, const float* __restrict__ Wr,
                                                        const float* __restrict__ bias, int T, int H, int E, int k,
                                                        float drop, int32_t* __restrict__ ids,
                                                        float* __restrict__ wout) {
    extern __shared__ __align__(16) uint8_t smem[];
    float* lg = (float*)smem;                  // [RT][E]
    float* xs = lg + kRouteF32Rows * E;        // [RT][chunk]
    const int t0 = blockIdx.x * kRouteF32Rows;
    const int wave = threadIdx.x / kWave;
    for (int e0 = 0; e0 < E; e0 += 256) {
        const int e = e0 + threadIdx.x;
        float acc[kRouteF32Rows];
#pragma unroll
        for (int m = 0; m < kRouteF32Rows; ++m) acc[m] = 0.0f;
        for (int h0 = 0; h0 < H; h0 += kRouteF32Chunk) {
            __syncthreads();
            for (int i = threadIdx.x; i < kRouteF32Rows * kRouteF32Chunk; i += 256) {
                const int m = i / kRouteF32Chunk, hh = i % kRouteF32Chunk;
                const int t = t0 + m, h = h0 + hh;
                xs[i] = (t < T && h < H) ? x[(long)t * H + h] : 0.0f;
            }
            __syncthreads();
            if (e < E) {
                const int hn = min(kRouteF32Chunk, H - h0);
                for (int hh = 0; hh < hn; ++hh) {
                    const float wv = Wr[(long)(h0 + hh) * E + e];
#pragma unroll
                    for (int m = 0; m < kRouteF32Rows; ++m) acc[m] = fmaf(xs[m * kRouteF32Chunk + hh], wv, acc[m]);
                }
            }
        }
        if (e < E) {
            const float b = bias ? bias[e] : 0.0f;
#pragma unroll
            for (int m = 0; m < kRouteF32Rows; ++m) lg[m * E + e] = acc[m] + b;
        }
    }
    __syncthreads();
    for (int m = wave; m < kRouteF32Rows; m += 4) {
        const long t = t0 + m;
        if (t < T) topk_one_token(lg + m * E, E, k, drop, t, ids, wout);
    }
}

// ---------------------------------------------------------------------------
// Pipelined router (bf16, E % 8 == 0, E <= 256, H % 64 == 0): 32 tokens per
// workgroup, the H loop streamed through a 3-stage direct-to-LDS ring (x rows
// k-contiguous, Wr rows n-contiguous and read k-packed with LDS transpose
// reads, as in the grouped GEMM). When the token blocks alone cannot fill the
// GPU, the H loop is split across S workgroups that write fp32 partial logits;
// a second kernel adds the S partials in a fixed order (reproducible) and runs
// the top-k.
constexpr int kR2Rows = 32;
constexpr int kR2BK = 64;
constexpr int kR2Stages = 3;

// RG row groups of 32 tokens share each Wr stage (4 waves per group): with
// RG = 2 a workgroup reads each Wr slice once for 64 tokens, halving the Wr
// traffic from L2, which dominates the router's loads at large T.
template <int EP, int RG = 1>
struct R2 {
    static constexpr int NWV = 4 * RG, ROWS = kR2Rows * RG;  // waves, tokens per workgroup
    static constexpr int A_BYTES = ROWS * kR2BK * 2;          // 4 KiB per group: one chunk per wave
    static constexpr int B_BYTES = kR2BK * EP * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int B_CHUNKS = B_BYTES / (1024 * NWV);  // per wave
    static constexpr int LOADS = 1 + B_CHUNKS;
    static constexpr int B_RCH = EP / 8;                     // 16-byte chunks per Wr row
    static constexpr int B_RPK = 1024 / (EP * 2);            // Wr rows per KiB
    static constexpr int NT = EP / 16;                       // 16-column MFMA tiles
    static constexpr int NTW = (NT + 3) / 4;                 // tiles per wave
    static constexpr int LDS = (kR2Stages * STAGE > ROWS * EP * 4) ? kR2Stages * STAGE : ROWS * EP * 4;
    static_assert(B_BYTES % (1024 * NWV) == 0 && B_CHUNKS >= 1, "Wr tile must be whole KiB chunks per wave");
    __device__ static int swz_b(int r, int c) { return EP >= 128 ? dma::swz_b(r, c) : c; }
};

template <int EP, bool SPLIT, int RG = 1>
__global__ __launch_bounds__(256 * RG) void route_v2_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wr,
                                                       const float* __restrict__ bias, int T, int H, int E, int k,
                                                       float drop, int steps_per_split, int32_t* __restrict__ ids,
                                                       float* __restrict__ wout, float* __restrict__ partial) {
    using C = R2<EP, RG>;
    __shared__ __align__(1024) uint8_t smem[C::LDS];
    const int t0 = blockIdx.x * C::ROWS;
    const int sp = blockIdx.y;
    const int wave = threadIdx.x / kWave, l = lane_id();
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const int rg = uwave / 4, wq = wave % 4;  // this wave's row group and its place in the group
    const int kbase = sp * steps_per_split * kR2BK;

    // global sources of this lane's LDS chunks
    const int arow = 8 * uwave + (l >> 3);
    const uint16_t* a_src = x + (long)min(t0 + arow, T - 1) * H + kbase + dma::swz_a(arow, l & 7) * 8;
    const uint16_t* b_src[C::B_CHUNKS];
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; ++i) {
        const int c = uwave + C::NWV * i;
        const int row = c * C::B_RPK + l / C::B_RCH;
        const int col = min(C::swz_b(row, l % C::B_RCH) * 8, E - 8);
        b_src[i] = Wr + (long)(kbase + row) * E + col;
    }
    dma::lds_u8* ring = (dma::lds_u8*)smem;
    auto issue = [&](int stage, int k0) {
        const uint32_t b0 = (uint32_t)(uintptr_t)(ring + stage * C::STAGE) + uwave * 1024;
        dma::lds_dma16(a_src + k0, b0);
#pragma unroll
        for (int i = 0; i < C::B_CHUNKS; ++i)
            dma::lds_dma16(b_src[i] + (long)k0 * E, b0 + C::A_BYTES + i * 1024 * C::NWV);
    };

    f32x4 acc[2][C::NTW];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < C::NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](dma::lds_u8* As) {
        dma::lds_u8* Bs = As + C::A_BYTES;
#pragma unroll
        for (int kk = 0; kk < kR2BK; kk += 32) {
            bf16x8 af[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = rg * 32 + i * 16 + (l & 15);
                af[i] = *(dma::lds_bf16x8*)(As + row * (kR2BK * 2) + dma::swz_a(row, (kk >> 3) + (l >> 4)) * 16);
            }
#pragma unroll
            for (int j = 0; j < C::NTW; ++j) {
                const int nt = wq + 4 * j;
                if (nt < C::NT) {
                    const int n = nt * 16 + 4 * (l & 3);
                    const int c = n >> 3, half = (n >> 2) & 1;
                    dma::s16x4 v[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int r = kk + 8 * (l >> 4) + 4 * h + ((l & 15) >> 2);
                        v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (dma::lds_s16x4*)(Bs + r * (EP * 2) + C::swz_b(r, c) * 16 + half * 8));
                    }
                    typedef __attribute__((ext_vector_type(8))) short s16x8;
                    const bf16x8 bfr = __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr, acc[i][j], 0, 0, 0);
                }
            }
        }
    };

    const int nsteps = steps_per_split;
    issue(0, 0);
    if (nsteps > 1) issue(1, kR2BK);
    for (int s = 0; s < nsteps; ++s) {
        if (s + 1 < nsteps) __builtin_amdgcn_s_waitcnt(dma::VmWait<C::LOADS>::value);
        else __builtin_amdgcn_s_waitcnt(dma::VmWait<0>::value);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (s + 2 < nsteps) issue((s + 2) % kR2Stages, (s + 2) * kR2BK);
        compute(ring + (s % kR2Stages) * C::STAGE);
    }

    if (SPLIT) {
        // partial[sp][t][e], e over all EP columns (columns >= E are ignored later)
#pragma unroll
        for (int j = 0; j < C::NTW; ++j) {
            const int nt = wq + 4 * j;
            if (nt < C::NT) {
                const int e = nt * 16 + (l & 15);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int t = t0 + rg * 32 + i * 16 + (l >> 4) * 4 + q;
                        if (t < T) partial[((long)sp * T + t) * EP + e] = acc[i][j][q];
                    }
            }
        }
        return;
    }
    asm volatile("" ::: "memory");
    __syncthreads();  // all waves done with the ring before it holds logits
    float* lg = (float*)smem;
#pragma unroll
    for (int j = 0; j < C::NTW; ++j) {
        const int nt = wq + 4 * j;
        if (nt < C::NT) {
            const int e = nt * 16 + (l & 15);
            const float b = (bias != nullptr && e < E) ? bias[e] : 0.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) lg[(rg * 32 + i * 16 + (l >> 4) * 4 + q) * EP + e] = acc[i][j][q] + b;
        }
    }
    __syncthreads();
    for (int m = wave; m < C::ROWS; m += C::NWV) {
        const long t = t0 + m;
        if (t < T) topk_select<(EP + kWave - 1) / kWave>(lg + m * EP, E, k, drop, t, ids, wout);
    }
}

// Sum the S partial logit rows of a token in split order, add the bias, top-k.
// Two shapes, both issuing their loads several at a time (a serial walk over
// S pays one L2/MALL round trip per split):
//  - route_reduce_wave_kernel, few splits (large T): one wave per token, lane
//    l owns experts l, l+64, ...; four splits' loads are in flight at once.
//  - route_reduce_block_kernel, many splits (small T, long H): one workgroup
//    per token; thread i owns expert i % EP and splits r, r+R, r+2R, ...
//    (r = i / EP, R = 256 / EP), eight loads in flight; the R partial sums are
//    then added in r order.
// Each order is fixed, so the logits are deterministic.
template <int EP>
__global__ __launch_bounds__(256) void route_reduce_wave_kernel(const float* __restrict__ partial, int S, int T,
                                                                const float* __restrict__ bias, int E, int k,
                                                                float drop, int32_t* __restrict__ ids,
                                                                float* __restrict__ wout) {
    constexpr int Q = (EP + kWave - 1) / kWave;
    __shared__ float lg[4][EP];
    const int wave = threadIdx.x / kWave, l = lane_id();
    const long t = (long)blockIdx.x * 4 + wave;
    if (t >= T) return;  // wave-uniform; no barrier follows
    const float* p = partial + t * EP;
    const long step = (long)T * EP;  // one split further
    float acc[Q];
#pragma unroll
    for (int j = 0; j < Q; ++j) acc[j] = 0.0f;
    int sp = 0;
    for (; sp + 4 <= S; sp += 4) {
        float q[4][Q];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < Q; ++j) {
                const int e = j * kWave + l;
                q[u][j] = e < EP ? p[(long)(sp + u) * step + e] : 0.0f;
            }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < Q; ++j) acc[j] += q[u][j];
    }
    for (; sp < S; ++sp)
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            const int e = j * kWave + l;
            if (e < EP) acc[j] += p[(long)sp * step + e];
        }
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        const int e = j * kWave + l;
        if (e < E) lg[wave][e] = acc[j] + (bias != nullptr ? bias[e] : 0.0f);
    }
    topk_select<(EP + kWave - 1) / kWave>(lg[wave], E, k, drop, t, ids, wout);
}

template <int EP>
__global__ __launch_bounds__(256) void route_reduce_block_kernel(const float* __restrict__ partial, int S, int T,
                                                                 const float* __restrict__ bias, int E, int k,
                                                                 float drop, int32_t* __restrict__ ids,
                                                                 float* __restrict__ wout) {
    constexpr int R = 256 / EP;
    __shared__ float part[R][EP];
    __shared__ float lg[EP];
    const long t = blockIdx.x;
    const int e = threadIdx.x % EP, r = threadIdx.x / EP;
    const float* p = partial + t * EP + e;
    const long step = (long)T * EP;
    float v = 0.0f;
    int sp = r;
    for (; sp + 7 * R < S; sp += 8 * R) {
        float q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) q[u] = p[(long)(sp + u * R) * step];
#pragma unroll
        for (int u = 0; u < 8; ++u) v += q[u];
    }
    for (; sp < S; sp += R) v += p[(long)sp * step];
    part[r][e] = v;
    __syncthreads();
    if (threadIdx.x >= kWave) return;  // wave 0 finishes; no barrier follows
    for (int j = threadIdx.x; j < E; j += kWave) {
        float sum = 0.0f;
#pragma unroll
        for (int rr = 0; rr < R; ++rr) sum += part[rr][j];
        lg[j] = sum + (bias != nullptr ? bias[j] : 0.0f);
    }
    topk_select<(EP + kWave - 1) / kWave, true>(lg, E, k, drop, t, ids, wout);  // few tokens: early exit pays
}

// Splits of the H loop: the smallest power of two that gives >= 512
// workgroups (two per CU, for enough loads in flight) and divides the number
// of 64-wide k-steps. Measured at T=8192, H=2048, E=128: router 21.5 us with
// two splits, 26.3 us with four (1024 workgroups), 34 us unsplit.
inline int route_splits(int T, int H) {
    const int blocks = (T + kR2Rows - 1) / kR2Rows;
    const int steps = H / kR2BK;
    int S = 1;
    while (blocks * S < 512 && S * 2 <= steps && steps % (S * 2) == 0) S *= 2;
    return S;
}

inline int route_ep(int E) { return E <= 32 ? 32 : E <= 64 ? 64 : E <= 128 ? 128 : 256; }

template <int EP>
hipError_t launch_v2(const uint16_t* x, const uint16_t* Wr, const float* bias, int T, int H, int E, int k, float drop,
                     int32_t* ids, float* w, float* partial, hipStream_t s) {
    const int S = route_splits(T, H);  // the split the workspace is sized for
    const int steps = H / kR2BK / S;
    // many tokens: 64 per workgroup (two row groups on one Wr stage, 8 waves), so the same number of waves
    // reads half as much of Wr from L2
    constexpr int RG2 = EP >= 64 ? 2 : 1;  // a Wr stage splits into whole KiB chunks over 8 waves from EP = 64
    const bool pair = RG2 == 2 && T >= 4096;
    const int rows = pair ? 2 * kR2Rows : kR2Rows;
    const dim3 grid((T + rows - 1) / rows, S);
    if (S == 1) {
        if (pair)
            hipLaunchKernelGGL((route_v2_kernel<EP, false, RG2>), grid, dim3(256 * RG2), 0, s, x, Wr, bias, T, H, E, k,
                               drop, steps, ids, w, (float*)nullptr);
        else
            hipLaunchKernelGGL((route_v2_kernel<EP, false>), grid, dim3(256), 0, s, x, Wr, bias, T, H, E, k, drop,
                               steps, ids, w, (float*)nullptr);
        return hipGetLastError();
    }
    if (pair)
        hipLaunchKernelGGL((route_v2_kernel<EP, true, RG2>), grid, dim3(256 * RG2), 0, s, x, Wr, bias, T, H, E, k, drop,
                           steps, ids, w, partial);
    else
        hipLaunchKernelGGL((route_v2_kernel<EP, true>), grid, dim3(256), 0, s, x, Wr, bias, T, H, E, k, drop, steps,
                           ids, w, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (S >= 16)
        hipLaunchKernelGGL(route_reduce_block_kernel<EP>, dim3(T), dim3(256), 0, s, (const float*)partial, S, T, bias,
                           E, k, drop, ids, w);
    else
        hipLaunchKernelGGL(route_reduce_wave_kernel<EP>, dim3((T + 3) / 4), dim3(256), 0, s, (const float*)partial, S,
                           T, bias, E, k, drop, ids, w);
    return hipGetLastError();
}

inline bool route_v2_ok(int H, int E) { return E % 8 == 0 && E <= 256 && H % kR2BK == 0; }

template <int MT, int NTW>
hipError_t launch_bf16(const uint16_t* x, const uint16_t* Wr, const float* bias, int T, int H, int E, int k,
                       float drop, int32_t* ids, float* w, hipStream_t s) {
    constexpr int RT = MT * 16;
    const int EP = (E + 15) & ~15;
    const size_t tiles = (size_t)(RT + EP) * kRouteS * sizeof(uint16_t);
    const size_t logits = (size_t)RT * EP * sizeof(float);
    const size_t lds = tiles > logits ? tiles : logits;
    const int grid = (T + RT - 1) / RT;
    if (E % 8 == 0)
        hipLaunchKernelGGL((route_bf16_kernel<MT, NTW, true>), dim3(grid), dim3(256), lds, s, x, Wr, bias, T, H, E,
                           k, drop, ids, w);
    else
        hipLaunchKernelGGL((route_bf16_kernel<MT, NTW, false>), dim3(grid), dim3(256), lds, s, x, Wr, bias, T, H,
                           E, k, drop, ids, w);
    return hipGetLastError();
}

// logits[t*EP + e] = sum over the S partial rows (in split order) + bias[e]
// for e < E, 0 for the padding columns (capacity-limited selection input).
__global__ __launch_bounds__(256) void logits_sum_kernel(const float* __restrict__ partial, int S, int T, int EP,
                                                         const float* __restrict__ bias, int E,
                                                         float* __restrict__ logits) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    const long n = (long)T * EP;
    if (i >= n) return;
    const int e = (int)(i % EP);
    float v = 0.0f;
    for (int sp = 0; sp < S; ++sp) v += partial[sp * n + i];
    logits[i] = e < E ? v + (bias != nullptr ? bias[e] : 0.0f) : 0.0f;
}

template <int EP>
hipError_t launch_logits(const uint16_t* x, const uint16_t* Wr, const float* bias, int T, int H, int E,
                         float* logits, float* partial, hipStream_t s) {
    const int S = route_splits(T, H);
    const int steps = H / kR2BK / S;
    constexpr int RG2 = EP >= 64 ? 2 : 1;  // as launch_v2: 64 tokens per workgroup at large T
    const bool pair = RG2 == 2 && T >= 4096;
    const int rows = pair ? 2 * kR2Rows : kR2Rows;
    const dim3 grid((T + rows - 1) / rows, S);
    if (pair)
        hipLaunchKernelGGL((route_v2_kernel<EP, true, RG2>), grid, dim3(256 * RG2), 0, s, x, Wr, bias, T, H, E, 1,
                           0.0f, steps, (int32_t*)nullptr, (float*)nullptr, partial);
    else
        hipLaunchKernelGGL((route_v2_kernel<EP, true>), grid, dim3(256), 0, s, x, Wr, bias, T, H, E, 1, 0.0f, steps,
                           (int32_t*)nullptr, (float*)nullptr, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long n = (long)T * EP;
    hipLaunchKernelGGL(logits_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)partial, S,
                       T, EP, bias, E, logits);
    return hipGetLastError();
}

}  // namespace

bool route_logits_ok(int H, int E, Dtype dt) { return dt == kBF16 && route_v2_ok(H, E); }

int route_logits_ld(int E) { return route_ep(E); }

size_t route_logits_partial_bytes(int T, int H, int E) {
    return (size_t)route_splits(T, H) * T * route_ep(E) * sizeof(float);
}

hipError_t launch_route_logits(const void* x, const void* Wr, const float* bias, int T, int H, int E, float* logits,
                               void* partial, hipStream_t s) {
    const uint16_t* xb = (const uint16_t*)x;
    const uint16_t* wb = (const uint16_t*)Wr;
    float* part = (float*)partial;
    switch (route_ep(E)) {
        case 32: return launch_logits<32>(xb, wb, bias, T, H, E, logits, part, s);
        case 64: return launch_logits<64>(xb, wb, bias, T, H, E, logits, part, s);
        case 128: return launch_logits<128>(xb, wb, bias, T, H, E, logits, part, s);
        default: return launch_logits<256>(xb, wb, bias, T, H, E, logits, part, s);
    }
}

size_t route_workspace_bytes(int T, int H, int E, Dtype dt) {
    if (dt != kBF16 || !route_v2_ok(H, E)) return 0;
    const int S = route_splits(T, H);
    return S > 1 ? (size_t)S * T * route_ep(E) * sizeof(float) : 0;
}

hipError_t launch_route(const void* x, const void* Wr, const float* bias, int T, int H, int E, int k, float drop,
                        Dtype dt, int32_t* ids, float* w, void* ws, hipStream_t s) {
    if (dt == kBF16) {
        const uint16_t* xb = (const uint16_t*)x;
        const uint16_t* wb = (const uint16_t*)Wr;
        if (route_v2_ok(H, E)) {
            float* part = (float*)ws;
            switch (route_ep(E)) {
                case 32: return launch_v2<32>(xb, wb, bias, T, H, E, k, drop, ids, w, part, s);
                case 64: return launch_v2<64>(xb, wb, bias, T, H, E, k, drop, ids, w, part, s);
                case 128: return launch_v2<128>(xb, wb, bias, T, H, E, k, drop, ids, w, part, s);
                default: return launch_v2<256>(xb, wb, bias, T, H, E, k, drop, ids, w, part, s);
            }
        }
        const int ntiles = (E + 15) / 16;
        if (ntiles <= 8) return launch_bf16<2, 2>(xb, wb, bias, T, H, E, k, drop, ids, w, s);
        if (ntiles <= 16) return launch_bf16<2, 4>(xb, wb, bias, T, H, E, k, drop, ids, w, s);
        if (ntiles <= 32) return launch_bf16<1, 8>(xb, wb, bias, T, H, E, k, drop, ids, w, s);
        return launch_bf16<1, 16>(xb, wb, bias, T, H, E, k, drop, ids, w, s);
    }
    const size_t lds = (size_t)kRouteF32Rows * (E + kRouteF32Chunk) * sizeof(float);
    const int grid = (T + kRouteF32Rows - 1) / kRouteF32Rows;
    hipLaunchKernelGGL(route_f32_kernel, dim3(grid), dim3(256), lds, s, (const float*)x, (const float*)Wr, bias, T,
                       H, E, k, drop, ids, w);
    return hipGetLastError();
}

}  // namespace moe
