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

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float4* __restrict__ y_perm,
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
                // each y_perm value is read exactly once: non-temporal loads
                const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
                const f32x4 q0 = r >= 0 ? __builtin_nontemporal_load((const f32x4*)(y_perm + row + c0)) : z4;
                const f32x4 q1 = (r >= 0 && two) ? __builtin_nontemporal_load((const f32x4*)(y_perm + row + c1)) : z4;
                v0[u] = make_float4(q0[0], q0[1], q0[2], q0[3]);
                v1[u] = make_float4(q1[0], q1[1], q1[2], q1[3]);
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

// Block-scaled fp16 y_perm (the W2 epilogue of moe_forward): each thread owns
// 8 consecutive columns, inside one 32-column scale block, read per slot as
// one 16-byte load of their fp16 values and one byte of the block's power-of-
// two exponent s; v = fp16 * 2^s exactly in fp32, then the same fmaf sequence
// per value as the fp32 form.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_f16s_kernel(const u32x4* __restrict__ vals,
                                                           const int8_t* __restrict__ scales,
                                                           const int32_t* __restrict__ inv,
                                                           const float* __restrict__ w,
                                                           const float4* __restrict__ ysh, int H8, int k,
                                                           void* __restrict__ y) {
    const long t = blockIdx.x;
    const int H32 = H8 / 4;  // scale bytes per row
    for (int c = threadIdx.x; c < H8; c += 256) {
        float a[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += 8) {
            u32x4 vh[8];
            int sc[8];
            float ww[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u;
                const int r = j < k ? inv[t * k + j] : -1;
                ww[u] = r >= 0 ? w[t * k + j] : 0.0f;
                const long rr = r >= 0 ? r : 0;
                // each y_perm value is read exactly once: non-temporal loads
                vh[u] = r >= 0 ? __builtin_nontemporal_load(vals + rr * H8 + c) : u32x4{0u, 0u, 0u, 0u};
                sc[u] = r >= 0 ? (int)scales[rr * H32 + c / 4] : 0;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (j0 + u < k && ww[u] != 0.0f) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint16_t hb = (uint16_t)((vh[u][i >> 1] >> (16 * (i & 1))) & 0xffffu);
                        const float v = ldexpf((float)__builtin_bit_cast(_Float16, hb), sc[u]);
                        a[i] = fmaf(ww[u], v, a[i]);
                    }
                }
            }
        }
        if (ysh != nullptr) {
            const float4 s0 = ysh[(t * H8 + c) * 2], s1 = ysh[(t * H8 + c) * 2 + 1];
            a[0] += s0.x;
            a[1] += s0.y;
            a[2] += s0.z;
            a[3] += s0.w;
            a[4] += s1.x;
            a[5] += s1.y;
            a[6] += s1.z;
            a[7] += s1.w;
        }
        if (OUT_BF16) {
            const u32x4 pk = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(a[4], a[5]),
                              pack_bf16x2(a[6], a[7])};
            ((u32x4*)y)[t * H8 + c] = pk;
        } else {
            ((float4*)y)[(t * H8 + c) * 2] = make_float4(a[0], a[1], a[2], a[3]);
            ((float4*)y)[(t * H8 + c) * 2 + 1] = make_float4(a[4], a[5], a[6], a[7]);
        }
    }
}

template <bool PACKED>
hipError_t combine(const void* y_perm, long sc_off, const int32_t* inv, const float* w, const float* y_shared, int T,
                   int H, int k, Dtype out_dt, void* y, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if constexpr (PACKED) {
        const u32x4* vals = (const u32x4*)y_perm;
        const int8_t* sc = (const int8_t*)((const uint8_t*)y_perm + sc_off);  // the scale bytes after the fp16 values
        if (out_dt == kBF16)
            hipLaunchKernelGGL((combine_f16s_kernel<true>), dim3(T), dim3(256), 0, s, vals, sc, inv, w,
                               (const float4*)y_shared, H / 8, k, y);
        else
            hipLaunchKernelGGL((combine_f16s_kernel<false>), dim3(T), dim3(256), 0, s, vals, sc, inv, w,
                               (const float4*)y_shared, H / 8, k, y);
        return hipGetLastError();
    }
    const int H4 = H / 4;
    const float4* yp = (const float4*)y_perm;
    if (out_dt == kBF16)
        hipLaunchKernelGGL((combine_kernel<true>), dim3(T), dim3(256), 0, s, yp, inv, w, (const float4*)y_shared, H4,
                           k, y);
    else
        hipLaunchKernelGGL((combine_kernel<false>), dim3(T), dim3(256), 0, s, yp, inv, w, (const float4*)y_shared, H4,
                           k, y);
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
