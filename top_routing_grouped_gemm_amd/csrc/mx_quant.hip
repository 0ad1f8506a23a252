// MX fp8 quantisers: token rows (before dispatch) and expert weights, in the
// OCP microscaling format with E4M3 elements -- every 32 consecutive values
// along a product's reduction axis share one power-of-two scale
// 2^(floor(log2 amax) - 8), stored as a biased exponent byte (E8M0).
//
// This extends page 1's 8-bit resident experts ("MoE大模型的智能调度…",
// www.jsqmd.com/news/1091713, section 4.1) to the activations, so that both
// products of an expert run on the fp8 matrix cores with the block scales
// applied in hardware (gemm_mx.hpp).
//
// Layouts:
//   rows:    codes xq[T][H] (row-major bytes); scales xs[H/128][T][4]: the 4
//            bytes of token t's 128-value chunk c at (c*T + t)*4.
//   weights: W[E][K][N] -> codes in 16 KiB tiles [E][Npad/128][K/128][128 n][128 k]
//            (16-byte chunk c of column n at c ^ ((n >> 1) & 7)); scales
//            [E][K/128][Npad][4]. Columns at or past N: code 0, scale byte 127.
#include "fp8_codes.hpp"
#include "gemm_mx.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

using dma::kMxBK;
using dma::kMxTileBytes;
using dma::kMxTileN;
using dma::mx_swz;

__device__ __forceinline__ float load_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_f32(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }

// One thread per 4 consecutive values; 8 threads form a 32-value block and 32
// threads a 128-value chunk (H % 128 == 0 keeps chunks inside a row).
template <typename TIn>
__global__ __launch_bounds__(256) void mx_rows_kernel(const TIn* __restrict__ X, long n4, int T, int H,
                                                      uint32_t* __restrict__ Xq, uint32_t* __restrict__ Xs) {
    const long g = (long)blockIdx.x * 256 + threadIdx.x;
    if (g >= n4) return;  // n4 is a multiple of 32: whole chunks leave together
    const long i0 = 4 * g;
    const float v0 = load_f32(X + i0), v1 = load_f32(X + i0 + 1), v2 = load_f32(X + i0 + 2),
                v3 = load_f32(X + i0 + 3);
    float am = fmaxf(fmaxf(fabsf(v0), fabsf(v1)), fmaxf(fabsf(v2), fabsf(v3)));
    am = fmaxf(am, __shfl_xor(am, 1));
    am = fmaxf(am, __shfl_xor(am, 2));
    am = fmaxf(am, __shfl_xor(am, 4));
    const int x = mx_exponent(am);
    Xq[g] = mx_codes4(v0, v1, v2, v3, x);
    const int l = lane_id(), base = l & ~31;
    const uint32_t b = (uint32_t)(x + 127);
    const uint32_t dw = __shfl(b, base) | (__shfl(b, base + 8) << 8) | (__shfl(b, base + 16) << 16) |
                        (__shfl(b, base + 24) << 24);
    if ((l & 31) == 0) {
        const long t = i0 / H;
        const int c = (int)((i0 % H) / 128);
        Xs[(long)c * T + t] = dw;
    }
}

// One 128-column x 128-k tile per workgroup; thread (n, half) encodes 64 k of
// column n (two blocks) into the LDS image of the tile.
template <typename TIn>
__global__ __launch_bounds__(256) void mx_weight_kernel(const TIn* __restrict__ W, int K, int N, int NB,
                                                        uint8_t* __restrict__ Wq, uint8_t* __restrict__ Ws) {
    __shared__ __align__(16) uint8_t tile[kMxTileBytes];
    __shared__ uint32_t sc[kMxTileN];
    const int KB = K / kMxBK;
    const long b = blockIdx.x;
    const int kb = (int)(b % KB), nb = (int)((b / KB) % NB);
    const long e = b / ((long)KB * NB);
    const int t = threadIdx.x, nn = t % kMxTileN, half = t / kMxTileN;
    const int n = nb * kMxTileN + nn;
    const TIn* src = W + e * K * N + (long)(kb * kMxBK + 64 * half) * N + n;
    uint32_t sbytes = 0;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        float v[32];
#pragma unroll
        for (int kk = 0; kk < 32; ++kk) v[kk] = n < N ? load_f32(src + (long)(32 * blk + kk) * N) : 0.0f;
        float am = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 32; ++kk) am = fmaxf(am, fabsf(v[kk]));
        const int x = mx_exponent(am);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int k = 64 * half + 32 * blk + 4 * q;  // k inside the tile
            *(uint32_t*)(tile + nn * kMxBK + 16 * ((k / 16) ^ mx_swz(nn)) + k % 16) =
                mx_codes4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], x);
        }
        sbytes |= (uint32_t)(x + 127) << (8 * blk);
    }
    __shared__ uint32_t part[2][kMxTileN];
    part[half][nn] = sbytes;
    __syncthreads();
    if (t < kMxTileN) sc[t] = part[0][t] | (part[1][t] << 16);
    __syncthreads();
    u32x4* out = (u32x4*)(Wq + ((e * NB + nb) * KB + kb) * (long)kMxTileBytes);
    for (int i = t; i < kMxTileBytes / 16; i += 256) out[i] = ((const u32x4*)tile)[i];
    if (t < kMxTileN) ((uint32_t*)Ws)[(e * KB + kb) * (long)(NB * kMxTileN) + nb * kMxTileN + t] = sc[t];
}

}  // namespace

long mx_weight_bytes(int E, int K, int N) { return (long)E * ((N + kMxTileN - 1) / kMxTileN) * kMxTileN * K; }

long mx_weight_scale_bytes(int E, int K, int N) {
    return (long)E * (K / kMxBK) * ((N + kMxTileN - 1) / kMxTileN) * kMxTileN * 4;
}

hipError_t launch_quantize_mx_rows(const void* x, int T, int H, Dtype dt, uint8_t* xq, uint8_t* xs, hipStream_t s) {
    const long n4 = (long)T * H / 4;
    const long grid = (n4 + 255) / 256;
    if (dt == kBF16)
        hipLaunchKernelGGL((mx_rows_kernel<uint16_t>), dim3((unsigned)grid), dim3(256), 0, s, (const uint16_t*)x, n4,
                           T, H, (uint32_t*)xq, (uint32_t*)xs);
    else
        hipLaunchKernelGGL((mx_rows_kernel<float>), dim3((unsigned)grid), dim3(256), 0, s, (const float*)x, n4, T, H,
                           (uint32_t*)xq, (uint32_t*)xs);
    return hipGetLastError();
}

hipError_t launch_quantize_mx_weights(const void* W, int E, int K, int N, Dtype dt, uint8_t* Wq, uint8_t* Ws,
                                      hipStream_t s) {
    const int NB = (N + kMxTileN - 1) / kMxTileN;
    const long grid = (long)E * NB * (K / kMxBK);
    if (dt == kBF16)
        hipLaunchKernelGGL((mx_weight_kernel<uint16_t>), dim3((unsigned)grid), dim3(256), 0, s, (const uint16_t*)W, K,
                           N, NB, Wq, Ws);
    else
        hipLaunchKernelGGL((mx_weight_kernel<float>), dim3((unsigned)grid), dim3(256), 0, s, (const float*)W, K, N,
                           NB, Wq, Ws);
    return hipGetLastError();
}

}  // namespace moe
