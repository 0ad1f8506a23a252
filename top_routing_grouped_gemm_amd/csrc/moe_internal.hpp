// Internal launch interface between the C ABI (moe_api.hip) and the kernels.
// Every launcher only enqueues work on `s` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

enum Dtype { kF32 = 0, kBF16 = 1 };

constexpr int kDispatchChunk = 1024;  // assignments per dispatch workgroup (scan: 7.4 -> 4.8 us at 65,536 vs 256)
constexpr int kSmallAssign = 1024;   // batches up to this many assignments dispatch in one workgroup

// Ragged GEMM tile shapes, chosen on the host from the mean rows per expert.
// kTileMixed: groups of very different sizes (mean 24..95 rows); the weight-
// streaming shape takes groups under kStreamRows rows, the large shape the rest.
enum TileCfg { kTileM16 = 0, kTileM64 = 1, kTileM128 = 2, kTileMixed = 3 };
constexpr int kStreamRows = 32;

inline int dispatch_blocks(long n_assign) { return (int)((n_assign + kDispatchChunk - 1) / kDispatchChunk); }

// Router workspace (fp32 partial logits when the H loop is split); 0 when none is needed.
size_t route_workspace_bytes(int T, int H, int E, Dtype dt);
// fp32 router logits (x@Wr + bias) to logits[T][route_logits_ld(E)] (bf16
// inputs, the direct-to-LDS router shapes only); partial holds
// route_logits_partial_bytes of split sums.
bool route_logits_ok(int H, int E, Dtype dt);
int route_logits_ld(int E);
size_t route_logits_partial_bytes(int T, int H, int E);
hipError_t launch_route_logits(const void* x, const void* Wr, const float* bias, int T, int H, int E, float* logits,
                               void* partial, hipStream_t s);
// Capacity-limited top-k selection on fp32 logits [T][ld] (see capacity.hip).
constexpr int kCapMaxRounds = 16;
size_t capacity_workspace_bytes(int T, int E);
hipError_t launch_capacity_select(const float* logits, int ld, int T, int E, int k, int cap, float drop,
                                  int32_t* ids, float* w, void* ws, hipStream_t s);
hipError_t launch_route(const void* x, const void* Wr, const float* bias, int T, int H, int E, int k,
                        float drop, Dtype dt, int32_t* ids, float* w, void* ws, hipStream_t s);

// Dispatch of more than kSmallAssign assignments, two passes: per-chunk
// expert histograms and in-chunk ranks (inv holds the rank in between), then
// every chunk's rows from the histograms. Used while chunks x experts <=
// kFinalizeCounts (each finalize workgroup reads all the counts).
constexpr long kFinalizeCounts = 32768;
bool dispatch_two_pass(long n_assign, int E);
hipError_t launch_count_rank(const int32_t* ids, const float* w, int n_assign, int E, int32_t* partial, int32_t* inv,
                             hipStream_t s);
hipError_t launch_finalize(const int32_t* ids, const int32_t* partial, int n_assign, int k, int E, int32_t* offsets,
                           int32_t* row_token, int32_t* inv, hipStream_t s);
// Larger batches: per-chunk expert histograms -> one-workgroup scan -> stable ranks.
hipError_t launch_count(const int32_t* ids, const float* w, int n_assign, int E, int32_t* partial,
                        hipStream_t s);
hipError_t launch_scan(int32_t* partial, int n_blocks, int E, int32_t* offsets, hipStream_t s);
// Padded fixed-shape layout (ablation): C rows per expert.
hipError_t launch_pad_dispatch(const void* x, const int32_t* ids, const int32_t* offsets, const int32_t* row_token,
                               const int32_t* inv, int T, int k, int E, int C, int row_bytes, void* x_pad,
                               int32_t* inv_pad, hipStream_t s);
hipError_t launch_uniform_offsets(int32_t* offsets, int E, int C, hipStream_t s);
hipError_t launch_dispatch_small(const int32_t* ids, const float* w, int n_assign, int k, int E, int32_t* offsets,
                                 int32_t* row_token, int32_t* inv, hipStream_t s);
hipError_t launch_index(const int32_t* ids, const float* w, const int32_t* partial, int n_assign, int k,
                        int E, int32_t* row_token, int32_t* inv, hipStream_t s);
// x_perm[inv[t*k+j]] = x[t] for every kept slot (inv >= 0); row_bytes % 16 == 0.
hipError_t launch_copy_rows(const void* x, const int32_t* inv, int T, int k, int row_bytes, void* x_perm,
                            hipStream_t s);

// The shared expert as one more group of the routed launches: T rows of x
// against W1s into its own h (h_cap as h_blocked gives for T rows, 0 for
// row-major), then that h against W2s into fp32 y[T][H].
struct SharedGroup {
    const void *x, *W1s, *W2s;
    void* h;
    long h_cap;
    float* y;
    int T;
};
// Whether the routed launches of this tile shape can take the shared expert
// as one more group: bf16, Fs == F, the large direct-to-LDS tiles.
bool ffn_shared_merges(TileCfg cfg, int H, int F, int Fs, Dtype dt);

// Grouped FFN. Rows of group e are [offsets[e], offsets[e+1]); with offsets == NULL there
// is a single group of rows [0, fixed_rows) (the shared expert on its own).
// h_cap: 0 for a row-major h[rows, F]; > 0 (from h_blocked) for the k-blocked
// h[F/32][h_cap][32] that the W1 launch writes and the W2 launch reads.
// sh (nullable; offsets != NULL and ffn_shared_merges only): the shared expert
// as one more group of the same launch.
hipError_t launch_ffn_up(const void* A, const int32_t* offsets, int E, int fixed_rows, int max_rows,
                         const void* W1, int H, int F, Dtype dt, void* h, TileCfg cfg, long h_cap, hipStream_t s,
                         const SharedGroup* sh = nullptr);
hipError_t launch_ffn_down(const void* h, const int32_t* offsets, int E, int fixed_rows, int max_rows,
                           const void* W2, int F, int H, Dtype dt, float* y, TileCfg cfg, long h_cap, hipStream_t s,
                           const SharedGroup* sh = nullptr);
// W1 -> SiLU -> W2 in one launch with h kept in LDS (64-row tiles; bf16, F % 256 == 0, F <= 768,
// H % 256 == 0): y_perm [max_rows][H] fp32.
bool ffn_fused_ok(int H, int F, Dtype dt);
hipError_t launch_ffn_fused(const void* x_perm, const int32_t* offsets, int E, int max_rows, const void* W1,
                            const void* W2, int H, int F, float* y_perm, hipStream_t s);
// Row capacity for the k-blocked h (the large direct-to-LDS shape with bf16
// and F % 32 == 0), or 0 for row-major.
long h_blocked(TileCfg cfg, int H, int F, long cap, Dtype dt);
// Whether the W2 launch can write y_perm as block-scaled fp16 (the
// direct-to-LDS shapes, H % 32 == 0): fp16 values of v * 2^-s at
// planes[r*H + n] (2 bytes), the signed exponent s of row r's 32-column block
// at ((int8_t*)planes + cap*H*2)[r*(H/32) + n/32]; cap*H*(2 + 1/32) bytes.
bool ffn_down_packs(TileCfg cfg, int F, int H, Dtype dt);
hipError_t launch_ffn_down_packed(const void* h, const int32_t* offsets, int E, int max_rows, const void* W2, int F,
                                  int H, TileCfg cfg, long h_cap, void* y_planes, long cap, hipStream_t s,
                                  const SharedGroup* sh = nullptr);
TileCfg choose_tile(long rows, int groups);
// Whether the W1 launch for this tile shape can read token rows of x directly
// through the row -> token map (the permute copy is then not needed).
bool ffn_up_gathers(TileCfg cfg, int H, int F, Dtype dt);
hipError_t launch_ffn_up_gather(const void* x, const int32_t* row_token, const int32_t* offsets, int E, int max_rows,
                                const void* W1, int H, int F, TileCfg cfg, long h_cap, void* h, hipStream_t s,
                                const SharedGroup* sh = nullptr);

// fp8 expert weights (fp8_quant.hip): bytes of the tiled codes of E matrices
// [K][N], and the quantiser (scales[E][N] fp32, codes in the tiled layout).
long fp8_weight_bytes(int E, int K, int N);
hipError_t launch_quantize_fp8(const void* W, int E, int K, int N, Dtype dt, uint8_t* Wq, float* scales,
                               hipStream_t s);
// Grouped FFN on fp8 weights (bf16 activations): W1 [E][H][F] and W2 [E][F][H]
// as tiled codes with per-column scales. a_rows != NULL gathers the W1 A rows
// from x through the row -> token map; packed: y in the block-scaled fp16 form
// of ffn_down_packs, else fp32 y[rows][H].
bool ffn_fp8_ok(int H, int F);
hipError_t launch_ffn_up_fp8(const void* A, const int32_t* a_rows, const int32_t* offsets, int E, int max_rows,
                             const uint8_t* W1q, const float* s1, int H, int F, TileCfg cfg, void* h, hipStream_t s);
hipError_t launch_ffn_down_fp8(const void* h, const int32_t* offsets, int E, int max_rows, const uint8_t* W2q,
                               const float* s2, int F, int H, TileCfg cfg, bool packed, void* y, long cap,
                               hipStream_t s);

// MX fp8 (mx_quant.hip, gemm_mx.hpp). Rows: R rows of x to row-major codes
// [R][H] and scales [H/128][R][4]. Weights [E][K][N] to code tiles (mx_weight_bytes) + scales
// (mx_weight_scale_bytes). The W1 launch gathers row-major token codes
// xq[x_rows][H] through row_token and writes SiLU(h) as k-blocked MX codes hq[F/64][cap][64] + scales
// hs[F/128][cap][4]; the W2 launch writes y as fp32 [cap][H] or in the
// block-scaled fp16 form (packed). H, F multiples of 128.
long mx_weight_bytes(int E, int K, int N);
long mx_weight_scale_bytes(int E, int K, int N);
hipError_t launch_quantize_mx_rows(const void* x, long R, int H, Dtype dt, uint8_t* xq, uint8_t* xs, hipStream_t s);
hipError_t launch_quantize_mx_weights(const void* W, int E, int K, int N, Dtype dt, uint8_t* Wq, uint8_t* Ws,
                                      hipStream_t s);
bool ffn_mx_ok(int H, int F);
hipError_t launch_ffn_up_mx(const void* xq, const void* xs, long x_rows, const int32_t* row_token,
                            const int32_t* offsets, int E, int max_rows, const uint8_t* W1q, const uint8_t* W1s, int H,
                            int F, void* hq, void* hs, long cap, hipStream_t s);
hipError_t launch_ffn_down_mx(const void* hq, const void* hs, long cap, const int32_t* offsets, int E, int max_rows,
                              const uint8_t* W2q, const uint8_t* W2s, int F, int H, bool packed, void* y,
                              hipStream_t s);

// y_perm given in the block-scaled fp16 form of ffn_down_packs (cap = row capacity).
hipError_t launch_combine_packed(const void* y_planes, long cap, const int32_t* inv, const float* w,
                                 const float* y_shared, int T, int H, int k, Dtype out_dt, void* y, hipStream_t s);
// Measurement aids (calibrate.hip): a bare bf16 MFMA loop, a streaming read, the grouped FFN's k-step.
hipError_t launch_calibrate_mfma(int workgroups, int waves, int iters, int operands, float* sink, hipStream_t s);
hipError_t launch_calibrate_read(const void* buf, long bytes, int workgroups, float* sink, hipStream_t s);
hipError_t launch_calibrate_kstep(const void* src, long span, int workgroups, int steps, int mode, float* sink,
                                  hipStream_t s);

hipError_t launch_combine(const float* y_perm, const int32_t* inv, const float* w, const float* y_shared,
                          int T, int H, int k, Dtype out_dt, void* y, hipStream_t s);

}  // namespace moe
