/*
 * moe.h - C ABI of a single MoE feed-forward layer's forward pass on one
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (page 3, "跟随一个Token走完路由、分发、专家计算到合并和多机放置的整条路径",
 * m.lsln.cn/news/228042, section "MoE层的结构与token路由") is
 *
 *     y(x) = sum over e in S(x) of w_e(x) * E_e(x)
 *
 * where S(x) is the set of experts the router selects for token x, w_e(x)
 * their routing weights and E_e expert e. The steps follow the same page's
 * section "单机MoE执行流水线" (single-GPU pipeline): router scores, top-k,
 * permute token rows into one contiguous block per expert while recording an
 * inverse map, the grouped GEMM with the activation and the output
 * projection, then restore token order, apply the weights and accumulate.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is a DEVICE pointer unless stated otherwise,
 *   allocated and owned by the caller. The library never allocates, frees or
 *   synchronises; each call only enqueues kernels on `stream` and returns.
 * - Row-major layouts: x[T,H], Wr[H,E], W1[E,H,F], W2[E,F,H], W1s[H,Fs],
 *   W2s[Fs,H]. T tokens, H hidden width, F expert hidden width, E routed
 *   experts, k experts per token, Fs shared-expert hidden width.
 * - `dt` is the type of x, Wr and the expert weights: MOE_F32 (fp32
 *   arithmetic throughout) or MOE_BF16 (bf16 operands on the matrix cores,
 *   fp32 accumulation). Router logits, routing weights, the router bias,
 *   y_perm and y_shared are always fp32. The intermediate expert activation
 *   h is held in `dt`.
 * - Slots: topk_ids[t*k + j] lists the k experts of token t in ascending
 *   expert id; topk_w holds their weights. A slot removed by the drop
 *   threshold keeps its expert id and has weight exactly 0.0f; a kept slot
 *   always has a weight > 0. Dropped slots are not dispatched; moe_permute
 *   also treats a slot whose id lies outside [0, E) as dropped.
 * - Rows of the permuted matrices are ordered by (expert id, token id), so
 *   expert e owns rows [expert_offsets[e], expert_offsets[e+1]) and the
 *   result is unique and reproducible (no atomics decide any order).
 * - The number of kept assignments A = expert_offsets[E] <= T*k stays on the
 *   device. Buffers with a row per assignment have capacity T*k rows; rows at
 *   or after A are left untouched.
 * - Size limits, checked before anything is launched (MOE_ERR_UNSUPPORTED):
 *   H % 8 == 0 and F % 8 == 0 (16-byte rows), E <= 1024, k <= 32,
 *   T*k < 2^31, and for the shared expert Fs % 8 == 0.
 *
 * Errors: a call returns MOE_OK after enqueueing its kernels. Argument
 * errors return a negative status and enqueue nothing: bad sizes
 * (T, H, F, E < 1; k < 1 or k > E), a null required pointer, drop_thresh
 * outside [0, 1/k], an unknown dtype, or a workspace smaller than required.
 * A failed launch returns MOE_ERR_HIP. Faults inside kernels surface at the
 * caller's next synchronisation of `stream`.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,
    MOE_ERR_UNSUPPORTED = -2,
    MOE_ERR_WORKSPACE = -3,
    MOE_ERR_HIP = -4
} moe_status_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_strerror(int status);

/* Library version as "major.minor.patch" (static string). */
const char* moe_version(void);

/*
 * Bytes of device workspace that moe_forward needs for these sizes (Fs = 0:
 * no shared expert). It also covers the step-wise calls, whose own needs are
 * moe_route_workspace_bytes (0 when the router needs none),
 * moe_permute_workspace_bytes and moe_ffn_workspace_bytes.
 * Returns 0 for sizes the library rejects. Host-only; no device access.
 */
size_t moe_workspace_bytes(int T, int H, int F, int E, int k, int Fs, moe_dtype_t dt);
size_t moe_route_workspace_bytes(int T, int H, int E, moe_dtype_t dt);
size_t moe_permute_workspace_bytes(int T, int E, int k);
size_t moe_ffn_workspace_bytes(int T, int F, int E, int k, int Fs, moe_dtype_t dt);

/*
 * moe_route - router logits, top-k, softmax weights, optional drop.
 *
 * Page 1 ("MoE大模型的智能调度…", www.jsqmd.com/news/1091713), section 2.2,
 * routing layer: the router scores each expert, the top-k logits are turned
 * into weights by a softmax, and a weight under the threshold (0.05 there)
 * is zeroed before the rest are renormalised. Page 3, section
 * "单机MoE执行流水线": top-k keeps the chosen expert indices and weights.
 *
 *   logits[t,e] = sum_h x[t,h] * Wr[h,e] + bias[e]       (fp32)
 *   S_t         = k largest logits, ties to the lower expert id
 *   w           = softmax over S_t; if drop_thresh > 0, every w < drop_thresh
 *                 is set to 0 and the survivors are divided by their sum
 *
 * x: [T,H] dt. Wr: [H,E] dt. bias: [E] fp32 or NULL (zero).
 * drop_thresh: 0 disables the drop; otherwise in (0, 1/k].
 * Out: topk_ids [T,k] int32, topk_w [T,k] fp32 (slot order: ascending id).
 * ws: device workspace of moe_route_workspace_bytes(T,H,E,dt) bytes (fp32
 * partial logits when the H loop is split across workgroups because T alone
 * cannot fill the GPU; the partials are added in a fixed order, so results do
 * not depend on timing). May be NULL when that size is 0.
 */
int moe_route(const void* x, const void* Wr, const float* bias, int T, int H, int E, int k,
              float drop_thresh, moe_dtype_t dt, int32_t* topk_ids, float* topk_w, void* ws,
              size_t ws_bytes, hipStream_t stream);

/*
 * moe_route_capacity - router logits, then capacity-limited top-k, softmax
 * weights and optional drop.
 *
 * Page 1 ("MoE大模型的智能调度…", www.jsqmd.com/news/1091713), section 3.2,
 * second routing pitfall: each expert accepts at most
 * capacity = tokens * k / experts * 1.2 selections; an over-capacity expert's
 * logit is set to -inf for the excess tokens, which choose again.
 *
 *   cap = ceil(T * k / E * cap_factor)   (double precision, in that order;
 *                                         cap_factor is a double so that a
 *                                         factor such as 1.2 enters exactly
 *                                         as the caller's double holds it)
 *   tokens in ascending id each take the k largest logits among experts
 *   selected fewer than cap times by the tokens before them (ties to the
 *   lower id); weights and drop as in moe_route, over the final selection.
 *   Capacity counts selections, before the drop.
 *
 * Same x, Wr, bias, outputs and slot order as moe_route; the result is
 * deterministic. Needs bf16 inputs, E % 8 == 0, E <= 256, H % 64 == 0
 * (otherwise MOE_ERR_UNSUPPORTED). cap_factor in (0, 1e6]
 * (MOE_ERR_INVALID_ARG otherwise); MOE_ERR_UNSUPPORTED when
 * E - floor(T*k/cap) < k, i.e. some token could find fewer than k experts
 * with room. ws: moe_route_capacity_workspace_bytes(T,H,E,dt) bytes.
 */
size_t moe_route_capacity_workspace_bytes(int T, int H, int E, moe_dtype_t dt);
int moe_route_capacity(const void* x, const void* Wr, const float* bias, int T, int H, int E, int k,
                       float drop_thresh, double cap_factor, moe_dtype_t dt, int32_t* topk_ids,
                       float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_select_capacity - the capacity-limited selection, weights and drop of
 * moe_route_capacity on given fp32 logits [T,E] (row-major, device), with
 * the capacity cap given in selections (cap >= 1). Decisions compare the
 * logits exactly as given. Same outputs as moe_route. MOE_ERR_UNSUPPORTED
 * when E - floor(T*k/cap) < k. ws: moe_select_capacity_workspace_bytes(T,E).
 */
size_t moe_select_capacity_workspace_bytes(int T, int E);
int moe_select_capacity(const float* logits, int T, int E, int k, float drop_thresh, int cap,
                        int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * Padded fixed-shape layout - the alternative to the ragged grouped GEMM,
 * kept as an ablation that measures what the ragged scheduler saves.
 *
 * Page 3, section "单机MoE执行流水线": experts receive different row counts;
 * they can be padded to one shape for a fixed batched GEMM, or run ragged in
 * one grouped kernel (the path above).
 *
 * moe_pad_dispatch: from moe_permute's outputs, x_pad [E*C, H] dt with
 *   x_pad[e*C + i] = x[row_token[expert_offsets[e] + i]] for i < count_e,
 *   zero rows for count_e <= i < C; inv_pad [T*k]: e*C + i for a kept slot
 *   with i = its row inside expert e, -1 if dropped or i >= C (a capacity C
 *   below the largest count drops those rows). topk_ids as from moe_route.
 * moe_grouped_ffn_padded: y_pad [E*C, H] fp32 = every expert's FFN over its
 *   C rows (the grouped kernels with E uniform groups). moe_combine then
 *   takes (y_pad, inv_pad) in place of (y_perm, inv).
 * ws: moe_grouped_ffn_padded_workspace_bytes(E,C,H,F,dt) bytes.
 */
int moe_pad_dispatch(const void* x, const int32_t* topk_ids, const int32_t* expert_offsets,
                     const int32_t* row_token, const int32_t* inv, int T, int H, int E, int k, int C,
                     moe_dtype_t dt, void* x_pad, int32_t* inv_pad, hipStream_t stream);
size_t moe_grouped_ffn_padded_workspace_bytes(int E, int C, int H, int F, moe_dtype_t dt);
int moe_grouped_ffn_padded(const void* x_pad, const void* W1, const void* W2, int E, int C, int H, int F,
                           moe_dtype_t dt, float* y_pad, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_permute - dispatch: group the kept assignments by expert.
 *
 * Page 3, section "一个批次如何变成各专家专属的矩阵": each assignment carries a
 * token vector, an expert and a weight; assignments are grouped per expert
 * into matrices and the source token id is kept beside every row. Section
 * "单机MoE执行流水线": the permute reads token vectors, writes them in expert
 * order and records an inverse map for the combine.
 *
 * In:  x [T,H] dt; topk_ids, topk_w [T,k] as written by moe_route.
 * Out: x_perm [T*k, H] dt       x_perm[r] = x[row_token[r]]
 *      expert_offsets [E+1]     exclusive prefix sum of per-expert counts
 *      row_token [T*k]          source token of row r (r < A)
 *      inv [T*k]                inv[t*k+j] = row of slot j of token t, -1 if dropped
 * ws: device workspace of at least moe_permute_workspace_bytes(T,E,k) bytes.
 */
int moe_permute(const void* x, const int32_t* topk_ids, const float* topk_w, int T, int H, int E,
                int k, moe_dtype_t dt, void* x_perm, int32_t* expert_offsets, int32_t* row_token,
                int32_t* inv, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_grouped_ffn - every expert's two-layer FFN over its rows, one ragged
 * launch per layer.
 *
 * Page 1, section 2.2, expert layer: each expert is an independent two-layer
 * FFN with its own W1, W2. Page 3, section "单机MoE执行流水线": a grouped
 * GEMM runs several expert matrices with different row counts in one kernel
 * launch; the experts then apply their activation and output projection.
 *
 *   for each expert e and row r in [expert_offsets[e], expert_offsets[e+1]):
 *     h[r]      = silu(x_perm[r] @ W1[e])        silu(u) = u / (1 + exp(-u))
 *     y_perm[r] = h[r] @ W2[e]                   (fp32 out)
 *
 * Optional shared expert (page 3, section "MoE层的结构与token路由": a shared
 * expert is not scored by the router and every token passes through it):
 * when W1s != NULL, also y_shared[t] = silu(x[t] @ W1s) @ W2s for all t.
 *
 * x_perm [T*k,H] dt; expert_offsets [E+1] on the device; W1 [E,H,F];
 * W2 [E,F,H]; y_perm [T*k,H] fp32. x [T,H] dt, W1s [H,Fs], W2s [Fs,H] and
 * y_shared [T,H] fp32 are needed only with the shared expert (else NULL, Fs=0).
 * ws: at least moe_ffn_workspace_bytes(T,F,E,k,Fs,dt) bytes (holds h).
 */
int moe_grouped_ffn(const void* x_perm, const int32_t* expert_offsets, const void* W1,
                    const void* W2, int T, int H, int F, int E, int k, moe_dtype_t dt,
                    float* y_perm, const void* x, const void* W1s, const void* W2s, int Fs,
                    float* y_shared, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_grouped_ffn_fused - the grouped FFN in one launch with the hidden
 * activation h kept on chip (never written to device memory).
 *
 * Page 3, section "单机MoE执行流水线": kernel fusion merges operators that
 * would run as separate launches, so the intermediate activation need not go
 * back to memory; a fused kernel covers only some data types and shapes, and
 * the rest use the modular path.
 *
 *   y_perm[r] = silu(x_perm[r] @ W1[e]) @ W2[e]   for r in group e (fp32 out,
 *               bf16 products, fp32 accumulation, h rounded to bf16 as in
 *               moe_grouped_ffn)
 *
 * Covers dt = MOE_BF16 with F % 256 == 0, F <= 768 and H % 256 == 0 (each
 * 64-row tile's h, 64 x F bf16, must fit in LDS beside its weight ring);
 * other shapes return MOE_ERR_UNSUPPORTED (use moe_grouped_ffn). No
 * workspace and no shared expert. Arguments as moe_grouped_ffn: x_perm
 * [T*k,H], expert_offsets [E+1], W1 [E,H,F], W2 [E,F,H], y_perm [T*k,H] fp32
 * (rows >= expert_offsets[E] untouched). Kept beside the two-launch path for
 * comparison: every 64-row tile streams its expert's whole W1 and W2, which
 * at prefill costs more than the h round trip it saves.
 */
int moe_grouped_ffn_fused(const void* x_perm, const int32_t* expert_offsets, const void* W1,
                          const void* W2, int T, int H, int F, int E, int k, moe_dtype_t dt,
                          float* y_perm, hipStream_t stream);

/*
 * moe_combine - unpermute and route-weight combine.
 *
 * Page 1, section 2.2, fusion layer: the output is the gate-weighted sum of
 * the chosen experts' outputs. Page 3, section "一个批次如何变成各专家专属的矩阵":
 * a token's results are scaled by their weights and added; section
 * "单机MoE执行流水线": the inverse map restores token order first.
 *
 *   y[t] = sum_{j: inv[t*k+j] >= 0} topk_w[t*k+j] * y_perm[inv[t*k+j]]  (+ y_shared[t])
 *
 * accumulated in fp32 in slot order, then written as out_dt (MOE_F32 keeps
 * the accumulator; MOE_BF16 rounds it to nearest even).
 * y_perm [T*k,H] fp32; inv, topk_w [T,k]; y_shared [T,H] fp32 or NULL;
 * y [T,H] out_dt.
 */
int moe_combine(const float* y_perm, const int32_t* inv, const float* topk_w,
                const float* y_shared, int T, int H, int k, moe_dtype_t out_dt, void* y,
                hipStream_t stream);

/*
 * moe_forward - the whole layer: moe_route, moe_permute, moe_grouped_ffn
 * (with the shared expert when W1s != NULL) and moe_combine, enqueued on one
 * stream with no host synchronisation in between.
 *
 * y [T,H] out_dt. The debug outputs topk_ids, topk_w [T,k], expert_offsets
 * [E+1] and inv [T,k] may be NULL; when given they receive the same values
 * the step-wise calls would produce. ws: at least
 * moe_workspace_bytes(T,H,F,E,k,Fs,dt) bytes.
 *
 * Precision: when dt = MOE_BF16, H % 32 == 0 and the library runs the
 * routed W2 product on its direct-to-LDS GEMM shapes (picked from the rows
 * per expert and the sizes), the routed y_perm stays inside the workspace as
 * block-scaled fp16: per row and 32 columns a power of two puts the block
 * maximum in [2^14, 2^15), and each value is rounded to fp16 (error <= 2^-11
 * of its magnitude; <= 2^(s-25) for the values under fp16's normal range,
 * below 2^-28 of the block maximum). y then differs from the step-wise
 * (fp32 y_perm) result by at most 2^-11 * max|y_perm| * sum_j topk_w[t,j]
 * plus fp32 accumulation; everything else is as in the step-wise calls.
 */
int moe_forward(const void* x, const void* Wr, const float* bias, const void* W1, const void* W2,
                const void* W1s, const void* W2s, int Fs, int T, int H, int F, int E, int k,
                float drop_thresh, moe_dtype_t dt, void* y, moe_dtype_t out_dt,
                int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* inv,
                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_forward_noalloc - moe_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same kernels and results (bit-identical y and debug
 * outputs), with no workspace argument. Its intermediate buffers live in one
 * static device array of 64 MiB that the library holds on each GPU it runs
 * on until the process ends; the call allocates and frees nothing.
 *
 * Limit: the call returns MOE_ERR_UNSUPPORTED when its buffers do not fit
 * the 64 MiB. They take, rounded up to 256 bytes each: 16*T*k + 4*(E+1) +
 * 4*E*ceil(T*k/1024) bytes of routing maps; T*k*F*b bytes of expert
 * activation (b = 2 for MOE_BF16, 4 for MOE_F32) and T*Fs*b + 4*T*H for a
 * shared expert; y_perm at T*k*H*(2 + 1/32) bytes on the bf16 shapes whose
 * W2 launch packs it (moe_forward's precision note), else 4*T*k*H plus
 * T*k*H*b for x_perm where the W1 launch does not gather rows of x; and the
 * router's split partial sums (moe_route_workspace_bytes). With H = 2048,
 * F = 768, bf16, that is about 5.7 KiB per assignment: T*k up to about
 * 11,000.
 *
 * Every call on one GPU uses that GPU's array and leaves the last call's
 * contents in it; nothing in it needs to start at zero. Calls that overlap
 * on one GPU (concurrent streams, or threads enqueueing on different
 * streams) race on the array and must be serialised by the caller.
 * Arguments, outputs and the other errors are those of moe_forward; a
 * failure to find the array's device address returns MOE_ERR_HIP.
 */
int moe_forward_noalloc(const void* x, const void* Wr, const float* bias, const void* W1,
                        const void* W2, const void* W1s, const void* W2s, int Fs, int T, int H,
                        int F, int E, int k, float drop_thresh, moe_dtype_t dt, void* y,
                        moe_dtype_t out_dt, int32_t* topk_ids, float* topk_w,
                        int32_t* expert_offsets, int32_t* inv, hipStream_t stream);

/*
 * Low-precision experts: fp8 (OCP e4m3) expert weights.
 *
 * Page 1 ("MoE大模型的智能调度…", www.jsqmd.com/news/1091713), section 4.1
 * (model loading and memory budget): the experts kept resident store their
 * FFN weights in 8 bits, halving their memory. The 8-bit format here is OCP
 * fp8 e4m3 with one fp32 scale per expert and output column:
 *
 *   scale[e][n]   = max_k |W[e][k][n]| / 448        (1.0 for an all-zero column)
 *   code[e][k][n] = e4m3(W[e][k][n] / scale[e][n])  nearest, ties to even,
 *                                                   saturating at +-448
 *
 * both divisions IEEE fp32. The dequantised weight is scale * value(code):
 * the matrix cores take the codes widened exactly to bf16, and the scale
 * multiplies each column's fp32 sums.
 *
 * Tiled code layout of Wq (device memory, caller-owned, moe_fp8_weight_bytes
 * bytes): for each expert e, 8 KiB tiles of 128 columns x 64 k; tile
 * (nb, kb) starts at byte ((e*NB + nb)*(K/64) + kb)*8192, NB = ceil(N/128).
 * Inside a tile, the code of (n, k) (tile-relative) is at byte
 *     n*64 + ((k/8) ^ (((n >> 1) & 7) ^ ((n >> 4) & 1)))*8 + k%8.
 * Columns at or past N hold code 0.
 *
 * moe_fp8_weight_bytes: bytes of Wq for E matrices [K][N]; 0 when a size is
 *   < 1 or K % 64 != 0.
 * moe_quantize_fp8: W [E][K][N] dt, finite values -> Wq and scales [E][N]
 *   fp32. K % 64 == 0, else MOE_ERR_UNSUPPORTED. W1 [E,H,F] is quantised
 *   with (K, N) = (H, F), W2 [E,F,H] with (F, H).
 * moe_grouped_ffn_fp8: moe_grouped_ffn on the dequantised weights with bf16
 *   activations (x_perm bf16, h bf16, y_perm fp32) and no shared expert.
 *   H and F multiples of 64 and >= 128, else MOE_ERR_UNSUPPORTED.
 *   ws: moe_ffn_workspace_bytes(T,F,E,k,0,MOE_BF16) bytes.
 * moe_forward_fp8: moe_forward with these experts; x and Wr bf16 (the router
 *   keeps bf16 operands and fp32 logits), no shared expert. Outputs, debug
 *   outputs and workspace as moe_forward with Fs = 0, dt = MOE_BF16.
 */
size_t moe_fp8_weight_bytes(int E, int K, int N);
int moe_quantize_fp8(const void* W, int E, int K, int N, moe_dtype_t dt, uint8_t* Wq, float* scales,
                     hipStream_t stream);
int moe_grouped_ffn_fp8(const void* x_perm, const int32_t* expert_offsets, const uint8_t* W1q,
                        const float* W1_scale, const uint8_t* W2q, const float* W2_scale, int T, int H,
                        int F, int E, int k, float* y_perm, void* ws, size_t ws_bytes, hipStream_t stream);
int moe_forward_fp8(const void* x, const void* Wr, const float* bias, const uint8_t* W1q,
                    const float* W1_scale, const uint8_t* W2q, const float* W2_scale, int T, int H, int F,
                    int E, int k, float drop_thresh, void* y, moe_dtype_t out_dt, int32_t* topk_ids,
                    float* topk_w, int32_t* expert_offsets, int32_t* inv, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/*
 * MX fp8: activations as well as expert weights in 8 bits, on the fp8 matrix
 * cores (v_mfma_scale_f32_32x32x64_f8f6f4 applies the block scales).
 *
 * This extends page 1's 8-bit resident experts (section 4.1, above) to the
 * token rows: they are quantised before dispatch, and each expert's SiLU
 * output is re-quantised before its second product. Format: OCP MX with E4M3
 * elements -- every 32 consecutive values along a product's reduction axis
 * share one scale X = 2^(floor(log2 amax) - 8) (1 for an all-zero block,
 * exponent clamped to [-127, 127]), stored as the byte exponent + 127
 * (E8M0); each value becomes e4m3(V / X), nearest, ties to even, saturating
 * at 448 (so values in [448, 512)X clamp to 448X). V / X is exact in fp32.
 *
 * Layouts (device memory, caller-owned):
 *   weights W [E][K][N] -> Wq (moe_mxfp8_weight_bytes): per expert, 8 KiB
 *     tiles of 128 columns x 64 k, tile (nb, kb) at ((e*NB + nb)*(K/64) + kb)*8192,
 *     NB = ceil(N/128); inside a tile the code of (n, k) is at
 *     n*64 + ((k/16) ^ (((n >> 1) & 3) ^ ((n >> 3) & 1)))*16 + k%16.
 *   weight scales (moe_mxfp8_scale_bytes): byte of (e, n, 32-k block b) at
 *     ((e*(K/128) + b/4)*NB*128 + n)*4 + b%4. Columns at or past N: code 0,
 *     scale byte 127.
 *   rows x [T][H] -> xq [T][H] bytes (row-major) and x_scale: byte of
 *     (t, 32-value block b) at ((b/4)*T + t)*4 + b%4.
 *   h_codes (moe_grouped_ffn_mxfp8): k-blocked, code of (row r, column f) at
 *     ((f/64)*T*k + r)*64 + f%64; h_scale: byte of (r, block b) at
 *     ((b/4)*T*k + r)*4 + b%4.
 *
 * moe_quantize_mxfp8: K % 128 == 0 (else MOE_ERR_UNSUPPORTED); W1 [E,H,F]
 *   uses (K, N) = (H, F), W2 [E,F,H] uses (F, H).
 * moe_quantize_mxfp8_rows: H % 128 == 0.
 * moe_grouped_ffn_mxfp8: the two expert products on MX operands, step-wise:
 *   x [T,H] bf16 and row_token, expert_offsets from moe_permute; the token
 *   rows are quantised once (moe_quantize_mxfp8_rows, into ws:
 *   moe_grouped_ffn_mxfp8_workspace_bytes(T,H,k) bytes) and the first product
 *   gathers their codes through row_token; writes h_codes,
 *   h_scale (the MX codes of silu(x_row @ W1), layouts above) and y_perm
 *   [T*k][H] fp32 = dequantised h @ W2. The matrix cores round inside each
 *   64-k product block (measured: up to about 5e-5 of the sum of the
 *   products' magnitudes), so an h value within that distance of an E4M3
 *   rounding boundary may take the neighbouring code.
 * moe_forward_mxfp8: the layer with MX experts: the router on bf16 x (fp32
 *   logits) as in moe_forward; x quantised to MX before dispatch; per
 *   expert y_e = mxq(silu(mxq(x) @ W1)) @ W2 with mxq the MX quantisation of
 *   its argument along the product's reduction axis and W1, W2 the MX
 *   weights; combine as moe_forward. x and Wr bf16; H and F multiples of 128;
 *   no shared expert. ws: moe_mxfp8_workspace_bytes(T,H,F,E,k).
 */
size_t moe_mxfp8_weight_bytes(int E, int K, int N);
size_t moe_mxfp8_scale_bytes(int E, int K, int N);
int moe_quantize_mxfp8(const void* W, int E, int K, int N, moe_dtype_t dt, uint8_t* Wq, uint8_t* W_scale,
                       hipStream_t stream);
int moe_quantize_mxfp8_rows(const void* x, int T, int H, moe_dtype_t dt, uint8_t* xq, uint8_t* x_scale,
                            hipStream_t stream);
size_t moe_grouped_ffn_mxfp8_workspace_bytes(int T, int H, int k);
int moe_grouped_ffn_mxfp8(const void* x, const int32_t* row_token, const int32_t* expert_offsets,
                          const uint8_t* W1q, const uint8_t* W1_scale, const uint8_t* W2q,
                          const uint8_t* W2_scale, int T, int H, int F, int E, int k, uint8_t* h_codes,
                          uint8_t* h_scale, float* y_perm, void* ws, size_t ws_bytes, hipStream_t stream);
size_t moe_mxfp8_workspace_bytes(int T, int H, int F, int E, int k);
int moe_forward_mxfp8(const void* x, const void* Wr, const float* bias, const uint8_t* W1q,
                      const uint8_t* W1_scale, const uint8_t* W2q, const uint8_t* W2_scale, int T, int H,
                      int F, int E, int k, float drop_thresh, void* y, moe_dtype_t out_dt,
                      int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* inv, void* ws,
                      size_t ws_bytes, hipStream_t stream);

/*
 * Measurement aids (not steps of the layer): the practical ceilings against
 * which the layer's kernels are read.
 *
 * moe_calibrate_mfma_bf16: `workgroups` workgroups of `waves_per_workgroup`
 *   (1..8) waves; each wave issues iters x 8 independent
 *   v_mfma_f32_32x32x16_bf16 and nothing else, i.e.
 *   workgroups * waves_per_workgroup * iters * 8 * 32768 FLOP. operands 0:
 *   one fixed low-entropy operand pair for every MFMA; 1: each of the 8
 *   MFMAs its own pseudo-random bf16 operands (random signs and mantissas, as
 *   a GEMM's fragments have), which switch more bits and run slower. One
 *   float per thread goes to sink[workgroups * waves_per_workgroup * 64]
 *   (keeps the loop from being removed; the values mean nothing).
 * moe_calibrate_stream_read: reads `bytes` (a multiple of 16) of `buf` once
 *   with 16-byte loads from `workgroups` workgroups of 256 threads, one float
 *   per thread to sink[workgroups * 256].
 * moe_calibrate_gemm_kstep: `workgroups` workgroups of 512 threads each run
 *   `steps` k-steps of the grouped FFN's 256x256 tile (the main loop of its
 *   large tiles: 8 waves, a 4-stage ring of 32 KB stages, 16-byte and
 *   transpose LDS reads, 16 v_mfma_f32_32x32x16_bf16 per wave, one barrier),
 *   i.e. workgroups * steps * 4194304 FLOP, without the tile's epilogue.
 *   mode 0: on the LDS alone, filled once with pseudo-random bf16 (src
 *   unused, may be NULL); mode 1: each
 *   step's stage also filled by 16-byte direct-to-LDS loads from src at byte
 *   offsets modulo span (span >= 32768, a multiple of 16; the whole span is
 *   read), 32 KB per step per workgroup; mode 2: those loads alone. One float
 *   per thread to sink[workgroups * 512].
 * All return MOE_ERR_INVALID_ARG for sizes outside these ranges or a null
 * pointer, MOE_ERR_HIP if the launch fails.
 */
int moe_calibrate_mfma_bf16(int workgroups, int waves_per_workgroup, int iters, int operands, float* sink,
                            hipStream_t stream);
int moe_calibrate_stream_read(const void* buf, size_t bytes, int workgroups, float* sink, hipStream_t stream);
int moe_calibrate_gemm_kstep(const void* src, size_t span, int workgroups, int steps, int mode, float* sink,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
