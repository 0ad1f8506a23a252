// Combine: restore token order, weight each expert result and add them.
//
// Page 1 ("MoE大模型的智能调度…", www.jsqmd.com/news/1091713), section 2.2,
// fusion layer: the layer output is the routing-weight gated sum of the
// chosen experts' outputs. Page 3 (m.lsln.cn/news/228042), section
// "一个批次如何变成各专家专属的矩阵": each of a token's expert results is scaled
// by its weight and the scaled results are added (T1 = 0.7 E1 + 0.3 E3);
// section "单机MoE执行流水线": the inverse map restores token order first.
//
// One workgroup per token; each thread owns 4-float column groups and
// gathers the token's k expert rows through inv with 16-byte loads,
// accumulating in fp32 in slot order, then adds the shared expert's row.
// HBM-bound: A*H*4 bytes of y_perm read, T*H*b written.
#include "moe_common.hpp"
#include "moe_internal.hpp"

namespace moe {

namespace {

// Each thread owns up to two 4-float column groups (c and c + 256) and
// processes slots 8 at a time with every load of a chunk issued before any of
// its FMAs, so up to 16 row gathers are in flight per thread. Accumulation is
// fp32 in slot order; dropped slots (w == 0) add nothing.
template <bool OUT_BF16>
__device__ __forceinline__ void combine_store(float4 acc, void* __restrict__ y, long idx) {
    if (OUT_BF16) {
        u32x2 pk = {pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w)};
        ((u32x2*)y)[idx] = pk;
    } else {
        ((float4*)y)[idx] = acc;
    }
}

// Four consecutive y_perm values (group idx = row*H/4 + column/4): fp32, or
// the 24-bit planes written by the W2 epilogue (upper 16 bits, 8 bytes per
// group; next 8 bits, 4 bytes per group at lo_off bytes), reassembled exactly.
template <bool PACKED>
__device__ __forceinline__ float4 load4(const void* __restrict__ yp, long lo_off, long idx) {
    if constexpr (PACKED) {
        const u32x2 h = ((const u32x2*)yp)[idx];
        const uint32_t l = ((const uint32_t*)((const uint8_t*)yp + lo_off))[idx];
        return make_float4(__uint_as_float((h[0] << 16) | ((l & 0xffu) << 8)),
                           __uint_as_float((h[0] & 0xffff0000u) | (((l >> 8) & 0xffu) << 8)),
                           __uint_as_float((h[1] << 16) | (((l >> 16) & 0xffu) << 8)),
                           __uint_as_float((h[1] & 0xffff0000u) | ((l >> 24) << 8)));
    } else {
        return ((const float4*)yp)[idx];
    }
}

template <bool OUT_BF16, bool PACKED>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_perm, long lo_off,
                                                      const int32_t* __restrict__ inv, const float* __restrict__ w,
                                                      const float4* __restrict__ ysh, int H4, int k,
                                                      void* __restrict__ y) {
    const long t = blockIdx.x;
    for (int c0 = threadIdx.x; c0 < H4; c0 += 512) {
        const int c1 = c0 + 256;
        const bool two = c1 < H4;
        float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
        for (int j0 = 0; j0 < k; j0 += 8) {
            float4 v0[8], v1[8];
            float ww[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u;
                const int r = j < k ? inv[t * k + j] : -1;
                ww[u] = r >= 0 ? w[t * k + j] : 0.0f;
                const long row = (long)(r >= 0 ? r : 0) * H4;
                v0[u] = r >= 0 ? load4<PACKED>(y_perm, lo_off, row + c0) : make_float4(0.f, 0.f, 0.f, 0.f);
                v1[u] = (r >= 0 && two) ? load4<PACKED>(y_perm, lo_off, row + c1) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (j0 + u < k && ww[u] != 0.0f) {
                    a0.x = fmaf(ww[u], v0[u].x, a0.x);
                    a0.y = fmaf(ww[u], v0[u].y, a0.y);
                    a0.z = fmaf(ww[u], v0[u].z, a0.z);
                    a0.w = fmaf(ww[u], v0[u].w, a0.w);
                    a1.x = fmaf(ww[u], v1[u].x, a1.x);
                    a1.y = fmaf(ww[u], v1[u].y, a1.y);
                    a1.z = fmaf(ww[u], v1[u].z, a1.z);
                    a1.w = fmaf(ww[u], v1[u].w, a1.w);
                }
            }
        }
        if (ysh != nullptr) {
            const float4 s0 = ysh[t * H4 + c0];
            a0.x += s0.x;
            a0.y += s0.y;
            a0.z += s0.z;
            a0.w += s0.w;
            if (two) {
                const float4 s1 = ysh[t * H4 + c1];
                a1.x += s1.x;
                a1.y += s1.y;
                a1.z += s1.z;
                a1.w += s1.w;
            }
        }
        combine_store<OUT_BF16>(a0, y, t * H4 + c0);
        if (two) combine_store<OUT_BF16>(a1, y, t * H4 + c1);
    }
}

template <bool PACKED>
hipError_t combine(const void* y_perm, long lo_off, const int32_t* inv, const float* w, const float* y_shared, int T,
                   int H, int k, Dtype out_dt, void* y, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int H4 = H / 4;
    if (out_dt == kBF16)
        hipLaunchKernelGGL((combine_kernel<true, PACKED>), dim3(T), dim3(256), 0, s, y_perm, lo_off, inv, w,
                           (const float4*)y_shared, H4, k, y);
    else
        hipLaunchKernelGGL((combine_kernel<false, PACKED>), dim3(T), dim3(256), 0, s, y_perm, lo_off, inv, w,
                           (const float4*)y_shared, H4, k, y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const float* y_perm, const int32_t* inv, const float* w, const float* y_shared, int T,
                          int H, int k, Dtype out_dt, void* y, hipStream_t s) {
    return combine<false>(y_perm, 0, inv, w, y_shared, T, H, k, out_dt, y, s);
}

hipError_t launch_combine_packed(const void* y_planes, long cap, const int32_t* inv, const float* w,
                                 const float* y_shared, int T, int H, int k, Dtype out_dt, void* y, hipStream_t s) {
    return combine<true>(y_planes, cap * H * 2, inv, w, y_shared, T, H, k, out_dt, y, s);
}

}  // namespace moe
