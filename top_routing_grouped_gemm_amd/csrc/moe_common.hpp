// Shared device helpers for the gfx950 MoE-layer kernels: vector types,
// bf16 conversion, wave64 reductions and the launch helpers' error plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int kWave = 64;

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Pack two floats into a bf16x2 word (lo = a, hi = b), RNE: one v_cvt_pk_bf16_f32 on gfx950, the same bits
// as f32_to_bf16_bits for finite values.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) float f32x2_t;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Wave-wide sum of a float (butterfly over 64 lanes; every lane gets the sum).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Wave-wide inclusive prefix sum of an int over lanes 0..63.
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int l = lane_id();
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int u = __shfl_up(v, o, kWave);
        if (l >= o) v += u;
    }
    return v;
}

// SiLU(u) = u * sigmoid(u) = u / (1 + e^-u), with the hardware reciprocal
// (about 1 ulp) in place of an IEEE divide: the value is rounded to bf16 or
// fed to an fp32 contraction next, so the last bit does not matter, and the
// divide sequence would cost the GEMM epilogue ~10 VALU ops per element.
// Large negative u: e^-u = inf, rcp(inf) = 0, result -0.
__device__ __forceinline__ float silu_f32(float u) { return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }

}  // namespace moe
