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
//   rows:    codes row-major xq[R][H]; scales xs[H/128][R][4]: the 4 bytes of
//            row r's 128-value chunk c at (c*R + r)*4 (a gathered row's 4
//            bytes for a 128-k stage pair are one aligned dword).
//   weights: W[E][K][N] -> codes in 8 KiB tiles [E][Npad/128][K/64][128 n][64 k]
//            (16-byte chunk c of column n at c ^ mx_swz(n)); scales
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

// One wave per 8 rows x 128 columns: lane l takes 16 consecutive values of
// row r0 + l/8 (two lanes per 32-value block, eight per 128-value chunk), so
// a row's source bytes are one contiguous read and its codes one contiguous
// write; one lane per row writes the chunk's scale dword.
template <typename TIn>
__global__ __launch_bounds__(256) void mx_rows_kernel(const TIn* __restrict__ X, long R, int H,
                                                      uint8_t* __restrict__ Xq, uint32_t* __restrict__ Xs) {
    const int l = lane_id();
    const long wv = ((long)blockIdx.x * 256 + threadIdx.x) / kWave;  // wave index
    const int chunks = H / 128;
    const long r = (wv / chunks) * 8 + l / 8;
    const int c = (int)(wv % chunks);
    if (r >= R) return;  // whole 8-lane row groups leave together
    const int col = c * 128 + (l % 8) * 16;
    const TIn* src = X + r * H + col;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = load_f32(src + i);
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(v[i]));
    am = fmaxf(am, __shfl_xor(am, 1));  // the lane pair of this 32-value block
    const int x = mx_exponent(am);
    const u32x4 codes = {mx_codes4(v[0], v[1], v[2], v[3], x), mx_codes4(v[4], v[5], v[6], v[7], x),
                         mx_codes4(v[8], v[9], v[10], v[11], x), mx_codes4(v[12], v[13], v[14], v[15], x)};
    *(u32x4*)(Xq + r * H + col) = codes;
    const int base = l & ~7;
    const uint32_t b = (uint32_t)(x + 127);
    const uint32_t dw = __shfl(b, base) | (__shfl(b, base + 2) << 8) | (__shfl(b, base + 4) << 16) |
                        (__shfl(b, base + 6) << 24);
    if ((l & 7) == 0) Xs[(long)c * R + r] = dw;
}

// One 128-column x 64-k tile per workgroup; thread (n, half) encodes the
// 32-value block of column n in its half into the LDS image of the tile and
// writes that block's scale byte.
template <typename TIn>
__global__ __launch_bounds__(256) void mx_weight_kernel(const TIn* __restrict__ W, int K, int N, int NB,
                                                        uint8_t* __restrict__ Wq, uint8_t* __restrict__ Ws) {
    __shared__ __align__(16) uint8_t tile[kMxTileBytes];
    const int KB = K / kMxBK;
    const long b = blockIdx.x;
    const int kb = (int)(b % KB), nb = (int)((b / KB) % NB);
    const long e = b / ((long)KB * NB);
    const int t = threadIdx.x, nn = t % kMxTileN, half = t / kMxTileN;
    const int n = nb * kMxTileN + nn;
    const TIn* src = W + e * K * N + (long)(kb * kMxBK + 32 * half) * N + n;
    float v[32];
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) v[kk] = n < N ? load_f32(src + (long)kk * N) : 0.0f;
    float am = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) am = fmaxf(am, fabsf(v[kk]));
    const int x = mx_exponent(am);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int k = 32 * half + 4 * q;  // k inside the tile
        *(uint32_t*)(tile + nn * kMxBK + 16 * ((k / 16) ^ mx_swz(nn)) + k % 16) =
            mx_codes4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], x);
    }
    // scale byte of block 2*kb + half: byte (2*(kb%2) + half) of the 128-k dword of column n
    Ws[((e * (KB / 2) + kb / 2) * (long)(NB * kMxTileN) + n) * 4 + 2 * (kb % 2) + half] = (uint8_t)(x + 127);
    __syncthreads();
    u32x4* out = (u32x4*)(Wq + ((e * NB + nb) * KB + kb) * (long)kMxTileBytes);
    for (int i = t; i < kMxTileBytes / 16; i += 256) out[i] = ((const u32x4*)tile)[i];
}

}  // namespace

long mx_weight_bytes(int E, int K, int N) { return (long)E * ((N + kMxTileN - 1) / kMxTileN) * kMxTileN * K; }

long mx_weight_scale_bytes(int E, int K, int N) {
    return (long)E * (K / 128) * ((N + kMxTileN - 1) / kMxTileN) * kMxTileN * 4;
}

hipError_t launch_quantize_mx_rows(const void* x, long R, int H, Dtype dt, uint8_t* xq, uint8_t* xs, hipStream_t s) {
    const long waves = (R + 7) / 8 * (H / 128);
    const long grid = (waves + 3) / 4;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (dt == kBF16)
        hipLaunchKernelGGL((mx_rows_kernel<uint16_t>), dim3((unsigned)grid), dim3(256), 0, s, (const uint16_t*)x, R, H,
                           xq, (uint32_t*)xs);
    else
        hipLaunchKernelGGL((mx_rows_kernel<float>), dim3((unsigned)grid), dim3(256), 0, s, (const float*)x, R, H, xq,
                           (uint32_t*)xs);
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
