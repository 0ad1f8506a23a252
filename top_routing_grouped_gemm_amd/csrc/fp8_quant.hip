// fp8 (OCP e4m3) expert weights: per-expert, per-output-column scales and the
// tiled code layout the grouped GEMM streams.
//
// Page 1 ("MoE大模型的智能调度…", www.jsqmd.com/news/1091713), section 4.1
// (model loading and memory budget): the experts kept resident are stored in
// 8 bits, which halves their footprint. On MI355X the 8-bit format is OCP fp8
// e4m3: the GEMM widens codes to bf16 exactly in registers, so decode, which
// streams every weight once, reads half the bytes.
//
//   scale[e][n] = max_k |W[e][k][n]| / 448   (448 = largest finite e4m3; 1 for an all-zero column)
//   code[e][k][n] = e4m3(W[e][k][n] / scale[e][n]), round to nearest, ties to even, saturating
//
// Both divisions are IEEE float32 (correctly rounded), so the codes are a
// function of the float32 values alone. Codes are stored as 8 KiB tiles of
// 128 columns x 64 k (see f8_swz in gemm_dma.hpp): per expert
// [ceil(N/128)][K/64][128][64] bytes, columns past N holding code 0.
#include "fp8_codes.hpp"
#include "gemm_dma.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

using dma::f8_swz;
using dma::kF8TileBytes;
using dma::kF8TileK;
using dma::kF8TileN;

__device__ __forceinline__ float load_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_f32(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }

// scales[e][n]; grid (ceil(N/64), E), 256 threads: 64 columns x 4 k-phases.
template <typename TIn>
__global__ __launch_bounds__(256) void fp8_scale_kernel(const TIn* __restrict__ W, int K, int N,
                                                        float* __restrict__ scales) {
    __shared__ float red[4][64];
    const int e = blockIdx.y, c = threadIdx.x & 63, kq = threadIdx.x >> 6;
    const int n = blockIdx.x * 64 + c;
    float m = 0.0f;
    if (n < N) {
        const TIn* p = W + (long)e * K * N + n;
#pragma unroll 8
        for (int k = kq; k < K; k += 4) m = fmaxf(m, fabsf(load_f32(p + (long)k * N)));
    }
    red[kq][c] = m;
    __syncthreads();
    if (kq == 0 && n < N) {
        m = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
        const float s = __fdiv_rn(m, 448.0f);
        scales[(long)e * N + n] = s == 0.0f ? 1.0f : s;
    }
}

// One 128 x 64 code tile per workgroup: codes land in LDS at their swizzled
// place, then the 8 KiB tile goes out in 16-byte stores.
template <typename TIn>
__global__ __launch_bounds__(256) void fp8_pack_kernel(const TIn* __restrict__ W, const float* __restrict__ scales,
                                                       int K, int N, int NB, uint8_t* __restrict__ Wq) {
    __shared__ __align__(16) uint8_t tile[kF8TileBytes];
    __shared__ float sc[kF8TileN];
    const int KB = K / kF8TileK;
    const long b = blockIdx.x;
    const int kb = (int)(b % KB), nb = (int)((b / KB) % NB);
    const long e = b / ((long)KB * NB);
    const int n0 = nb * kF8TileN, k0 = kb * kF8TileK, t = threadIdx.x;
    if (t < kF8TileN) sc[t] = n0 + t < N ? scales[e * N + n0 + t] : 1.0f;
    __syncthreads();
    const TIn* We = W + e * K * N;
    for (int i = t; i < kF8TileBytes; i += 256) {
        const int kk = i / kF8TileN, nn = i % kF8TileN, n = n0 + nn;
        uint32_t code = 0;
        if (n < N) code = e4m3_rne(__fdiv_rn(load_f32(We + (long)(k0 + kk) * N + n), sc[nn]));
        tile[nn * kF8TileK + (((kk >> 3) ^ f8_swz(nn)) << 3) + (kk & 7)] = (uint8_t)code;
    }
    __syncthreads();
    u32x4* out = (u32x4*)(Wq + ((e * NB + nb) * KB + kb) * (long)kF8TileBytes);
    for (int i = t; i < kF8TileBytes / 16; i += 256) out[i] = ((const u32x4*)tile)[i];
}

template <typename TIn>
hipError_t run_quantize(const void* W, int E, int K, int N, uint8_t* Wq, float* scales, hipStream_t s) {
    const int NB = (N + kF8TileN - 1) / kF8TileN;
    hipLaunchKernelGGL((fp8_scale_kernel<TIn>), dim3((N + 63) / 64, E), dim3(256), 0, s, (const TIn*)W, K, N,
                       scales);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const long grid = (long)E * NB * (K / kF8TileK);
    hipLaunchKernelGGL((fp8_pack_kernel<TIn>), dim3((unsigned)grid), dim3(256), 0, s, (const TIn*)W, scales, K, N,
                       NB, Wq);
    return hipGetLastError();
}

}  // namespace

long fp8_weight_bytes(int E, int K, int N) {
    return (long)E * ((N + kF8TileN - 1) / kF8TileN) * kF8TileN * K;
}

hipError_t launch_quantize_fp8(const void* W, int E, int K, int N, Dtype dt, uint8_t* Wq, float* scales,
                               hipStream_t s) {
    if (dt == kBF16) return run_quantize<uint16_t>(W, E, K, N, Wq, scales, s);
    return run_quantize<float>(W, E, K, N, Wq, scales, s);
}

}  // namespace moe
