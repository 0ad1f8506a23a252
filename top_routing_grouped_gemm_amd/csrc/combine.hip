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

// Slots are processed 8 at a time with every load of a chunk issued before
// any of its FMAs, so one thread keeps up to 8 row gathers in flight.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float4* __restrict__ y_perm, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, const float4* __restrict__ ysh,
                                                      int H4, int k, void* __restrict__ y) {
    const long t = blockIdx.x;
    for (int c = threadIdx.x; c < H4; c += 256) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j0 = 0; j0 < k; j0 += 8) {
            float4 v[8];
            float ww[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u;
                const int r = j < k ? inv[t * k + j] : -1;
                ww[u] = r >= 0 ? w[t * k + j] : 0.0f;
                v[u] = r >= 0 ? y_perm[(long)r * H4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (j0 + u < k && ww[u] != 0.0f) {  // slot order; dropped slots add nothing
                    acc.x = fmaf(ww[u], v[u].x, acc.x);
                    acc.y = fmaf(ww[u], v[u].y, acc.y);
                    acc.z = fmaf(ww[u], v[u].z, acc.z);
                    acc.w = fmaf(ww[u], v[u].w, acc.w);
                }
            }
        }
        if (ysh != nullptr) {
            const float4 v = ysh[t * H4 + c];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        if (OUT_BF16) {
            u32x2 pk = {pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w)};
            ((u32x2*)y)[t * H4 + c] = pk;
        } else {
            ((float4*)y)[t * H4 + c] = acc;
        }
    }
}

}  // namespace

hipError_t launch_combine(const float* y_perm, const int32_t* inv, const float* w, const float* y_shared, int T,
                          int H, int k, Dtype out_dt, void* y, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int H4 = H / 4;
    if (out_dt == kBF16)
        hipLaunchKernelGGL(combine_kernel<true>, dim3(T), dim3(256), 0, s, (const float4*)y_perm, inv, w,
                           (const float4*)y_shared, H4, k, y);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3(T), dim3(256), 0, s, (const float4*)y_perm, inv, w,
                           (const float4*)y_shared, H4, k, y);
    return hipGetLastError();
}

}  // namespace moe
