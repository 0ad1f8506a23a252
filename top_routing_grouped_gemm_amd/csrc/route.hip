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
// top-k of one token at a time with wave64 shuffle reductions; the logits are
// never written to memory.
#include <float.h>
#include <math.h>

#include "mfma_tiles.hpp"
#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int kRouteBK = 32;
constexpr int kRouteS = kRouteBK + 8;  // LDS row stride (bf16 elements)
constexpr int kQMax = 16;              // experts per lane: E <= 1024

// Top-k of one token whose E logits sit in LDS at lg[0..E). Whole wave.
__device__ void topk_one_token(const float* lg, int E, int k, float drop, long t, int32_t* __restrict__ ids,
                               float* __restrict__ wout) {
    const int l = lane_id();
    float v[kQMax];
#pragma unroll
    for (int q = 0; q < kQMax; ++q) {
        const int e = q * kWave + l;
        v[q] = (e < E) ? lg[e] : -INFINITY;
    }
    int my_id = 0x7fffffff;
    float my_v = -INFINITY;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < kQMax; ++q) {
            const int e = q * kWave + l;
            if (e < E && (v[q] > bv || (v[q] == bv && e < bi))) {
                bv = v[q];
                bi = e;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, kWave);
            const int oi = __shfl_xor(bi, o, kWave);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if (l == j) {
            my_id = bi;
            my_v = bv;
        }
        if ((bi & (kWave - 1)) == l) {
            const int qs = bi / kWave;
#pragma unroll
            for (int q = 0; q < kQMax; ++q)
                if (q == qs) v[q] = -INFINITY;
        }
    }
    // softmax over the k selected logits; lane 0 holds the largest
    const float m = __shfl(my_v, 0, kWave);
    const bool sel = l < k;
    float p = sel ? expf(my_v - m) : 0.0f;
    float w = p / wave_sum(p);
    bool kept = sel;
    if (drop > 0.0f) {
        kept = sel && !(w < drop);
        const float wk = kept ? w : 0.0f;
        w = wk / wave_sum(wk);
    }
    if (kept) w = fmaxf(w, FLT_MIN);  // a kept slot never carries 0.0f
    // slot = rank of the expert id among the k selected
    int rank = 0;
    for (int i = 0; i < k; ++i) rank += (__shfl(my_id, i, kWave) < my_id);
    if (sel) {
        ids[t * k + rank] = my_id;
        wout[t * k + rank] = kept ? w : 0.0f;
    }
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

}  // namespace

hipError_t launch_route(const void* x, const void* Wr, const float* bias, int T, int H, int E, int k, float drop,
                        Dtype dt, int32_t* ids, float* w, hipStream_t s) {
    if (dt == kBF16) {
        const uint16_t* xb = (const uint16_t*)x;
        const uint16_t* wb = (const uint16_t*)Wr;
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
