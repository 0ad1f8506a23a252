// Dispatch: group the kept (token, expert) assignments by expert and copy
// token rows into one contiguous block per expert, recording the inverse map.
//
// Page 3 (m.lsln.cn/news/228042), section "一个批次如何变成各专家专属的矩阵":
// assignments are grouped per expert into matrices with the source token id
// kept beside every row, and an expert's batch counts assignments (k rows per
// token). Section "单机MoE执行流水线": the permute reads token vectors, writes
// them in expert order and records an inverse map for the combine.
//
// Order is fixed by (expert, token), never by atomics. Batches of at most
// 1024 assignments run count, scan and rank in one workgroup
// (dispatch_block.hpp). Larger ones take chunks of 1024 assignments:
//   count_rank - each workgroup histograms its chunk per expert and ranks
//            every assignment within its expert inside the chunk (wave
//            ballots match equal expert ids, LDS combines the 16 waves); the
//            rank goes to inv, the histogram to partial[chunk][expert];
//   finalize - each workgroup sums the histograms itself (the column sums give
//            the expert offsets, the sums over earlier chunks its chunk's
//            first row per expert), so no separate scan launch is needed, and
//            turns its chunk's ranks into rows: row_token and inv;
//   copy   - token-major: each token row is read once and written to its k
//            destination rows (HBM-bound: T*H*b read, A*H*b written).
// When chunks x experts is too large for every workgroup to read the
// histograms (more than kFinalizeCounts), one workgroup scans them instead
// (count, scan, index).
#include "dispatch_block.hpp"
#include "moe_common.hpp"
#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int kMaxE = 1024;
static_assert(kMaxE == kSmallAssign, "dispatch_small_kernel scans one expert per thread");

__global__ __launch_bounds__(kDispatchChunk) void count_kernel(const int32_t* __restrict__ ids,
                                                               const float* __restrict__ w, int n_assign, int E,
                                                               int32_t* __restrict__ partial) {
    __shared__ int hist[kMaxE];
    for (int e = threadIdx.x; e < E; e += kDispatchChunk) hist[e] = 0;
    __syncthreads();
    const int a = blockIdx.x * kDispatchChunk + threadIdx.x;
    if (a < n_assign && w[a] != 0.0f) {
        const int e = ids[a];
        if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);  // order-free: only a count
    }
    __syncthreads();
    int32_t* out = partial + (long)blockIdx.x * E;
    for (int e = threadIdx.x; e < E; e += kDispatchChunk) out[e] = hist[e];
}

// One workgroup of 1024 threads. partial[b][e] (counts) becomes the first
// output row of chunk b's assignments to expert e. Threads are arranged as
// G groups of E experts; group g owns a contiguous range of chunks, so the
// loads of a column walk are independent and can all be in flight at once.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ partial, int n_blocks, int E,
                                                    int32_t* __restrict__ offsets) {
    __shared__ int gs[1024];   // [G][E] per-group sums
    __shared__ int eoff[kMaxE];
    __shared__ int wsum[16];
    const int tid = threadIdx.x, l = lane_id(), wv = tid / kWave;
    const int G = (1024 / E) > 0 ? (1024 / E) : 1;
    const int bpg = (n_blocks + G - 1) / G;
    const int e = tid % E, g = tid / E;
    const bool act = tid < E * G;
    const int b0 = g * bpg, b1 = min(n_blocks, b0 + bpg);
    if (act) {
        int s = 0;
        for (int b = b0; b < b1; b += 16) {  // 16 independent loads in flight
            int c[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) c[u] = (b + u < b1) ? partial[(long)(b + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 16; ++u) s += c[u];
        }
        gs[g * E + e] = s;
    }
    __syncthreads();
    int v = 0;
    if (tid < E)
        for (int i = 0; i < G; ++i) v += gs[i * E + tid];
    const int incl = wave_incl_scan(v);
    if (l == kWave - 1) wsum[wv] = incl;
    __syncthreads();
    int wbase = 0;
    for (int i = 0; i < wv; ++i) wbase += wsum[i];
    const int excl = wbase + incl - v;
    if (tid < E) {
        eoff[tid] = excl;
        offsets[tid] = excl;
    }
    if (tid == E - 1) offsets[E] = excl + v;
    __syncthreads();
    if (act) {
        int run = eoff[e];
        for (int i = 0; i < g; ++i) run += gs[i * E + e];
        for (int b = b0; b < b1; b += 16) {
            int c[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) c[u] = (b + u < b1) ? partial[(long)(b + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (b + u < b1) {
                    partial[(long)(b + u) * E + e] = run;
                    run += c[u];
                }
        }
    }
}

__global__ __launch_bounds__(kDispatchChunk) void index_kernel(const int32_t* __restrict__ ids,
                                                               const float* __restrict__ w,
                                                               const int32_t* __restrict__ partial, int n_assign,
                                                               int k, int E, int ebits, int32_t* __restrict__ row_token,
                                                               int32_t* __restrict__ inv) {
    constexpr int NW = kDispatchChunk / kWave;
    __shared__ int wc[NW][kMaxE];
    const int tid = threadIdx.x, l = lane_id(), wv = tid / kWave;
    for (int i = tid; i < NW * E; i += kDispatchChunk) (&wc[0][0])[(i / E) * kMaxE + (i % E)] = 0;
    const int a = blockIdx.x * kDispatchChunk + tid;
    const bool valid = a < n_assign;
    const int id = valid ? ids[a] : 0;
    const bool kept = valid && w[a] != 0.0f && (unsigned)id < (unsigned)E;  // out-of-range ids: dropped
    const int e = kept ? id : 0;
    // lanes of this wave holding the same expert id: AND of per-bit ballots
    unsigned long long same = __ballot(kept);
    for (int b = 0; b < ebits; ++b) {
        const bool bit = (e >> b) & 1;
        const unsigned long long bal = __ballot(bit);
        same &= bit ? bal : ~bal;
    }
    const unsigned long long below = (l == 0) ? 0ull : (~0ull >> (kWave - l));
    const int rank = __popcll(same & below);
    const int cnt = __popcll(same);
    __syncthreads();
    if (kept && rank == 0) wc[wv][e] = cnt;
    __syncthreads();
    int r = -1;
    if (valid) {
        if (kept) {
            r = partial[(long)blockIdx.x * E + e] + rank;
            for (int i = 0; i < wv; ++i) r += wc[i][e];
            row_token[r] = a / k;
        }
        inv[a] = r;
    }
}

// The whole dispatch of a batch of at most kSmallAssign assignments in one
// workgroup (dispatch_block.hpp). Saves two launches where latency, not
// bandwidth, is the cost.
__global__ __launch_bounds__(kSmallAssign) void dispatch_small_kernel(const int32_t* __restrict__ ids,
                                                                      const float* __restrict__ w, int n_assign,
                                                                      int k, int E, int ebits,
                                                                      int32_t* __restrict__ offsets,
                                                                      int32_t* __restrict__ row_token,
                                                                      int32_t* __restrict__ inv) {
    __shared__ DispatchSmem sm;
    dispatch_whole(ids, w, n_assign, k, E, ebits, offsets, row_token, inv, sm);
}

// count_rank: chunk b = blockIdx.x of kDispatchChunk assignments. partial[b][e]
// = kept assignments of the chunk with expert e; inv[a] = rank of a among the
// chunk's assignments to its expert (token order), -1 when dropped.
__global__ __launch_bounds__(kDispatchChunk) void count_rank_kernel(const int32_t* __restrict__ ids,
                                                                    const float* __restrict__ w, int n_assign, int E,
                                                                    int ebits, int32_t* __restrict__ partial,
                                                                    int32_t* __restrict__ inv) {
    constexpr int NW = kDispatchChunk / kWave;
    __shared__ int wc[NW][kMaxE];
    const int tid = threadIdx.x, l = lane_id(), wv = tid / kWave;
    for (int i = tid; i < NW * E; i += kDispatchChunk) wc[i / E][i % E] = 0;
    const int a = blockIdx.x * kDispatchChunk + tid;
    const bool valid = a < n_assign;
    const int id = valid ? ids[a] : 0;
    const bool kept = valid && w[a] != 0.0f && (unsigned)id < (unsigned)E;  // out-of-range ids: dropped
    const int e = kept ? id : 0;
    unsigned long long same = __ballot(kept);
    for (int b = 0; b < ebits; ++b) {
        const bool bit = (e >> b) & 1;
        const unsigned long long bal = __ballot(bit);
        same &= bit ? bal : ~bal;
    }
    const unsigned long long below = (l == 0) ? 0ull : (~0ull >> (kWave - l));
    const int rank = __popcll(same & below);
    const int cnt = __popcll(same);
    __syncthreads();
    if (kept && rank == 0) wc[wv][e] = cnt;
    __syncthreads();
    int32_t* out = partial + (long)blockIdx.x * E;
    for (int x = tid; x < E; x += kDispatchChunk) {  // wave prefixes per expert, chunk totals
        int run = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int c = wc[i][x];
            wc[i][x] = run;
            run += c;
        }
        out[x] = run;
    }
    __syncthreads();
    if (valid) inv[a] = kept ? wc[wv][e] + rank : -1;
}

// finalize: chunk b = blockIdx.x. Thread (g, e) (G = 1024/E groups) sums
// column e of partial over its share of the chunks, all of them and those
// before b apart; a scan over e of the column totals gives the expert
// offsets. Then inv[a] (a rank) becomes offsets[e] + earlier chunks' count of
// e + rank, and row_token of that row the token of a. Workgroup 0 also writes
// offsets. Every workgroup reads the nb x E histogram (L2-resident).
__global__ __launch_bounds__(kDispatchChunk) void finalize_kernel(const int32_t* __restrict__ ids,
                                                                  const int32_t* __restrict__ partial, int nb,
                                                                  int n_assign, int k, int E,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ row_token,
                                                                  int32_t* __restrict__ inv) {
    constexpr int NW = kDispatchChunk / kWave;
    __shared__ int gall[kDispatchChunk];  // [G][E] column sums over a group's chunks
    __shared__ int gbef[kDispatchChunk];  // [G][E] the same over the group's chunks before b
    __shared__ int base[kMaxE];
    __shared__ int wsum[NW];
    const int tid = threadIdx.x, l = lane_id(), wv = tid / kWave;
    const int b = blockIdx.x;
    // this workgroup's assignment and its rank, loaded before the histogram walk
    const int a = b * kDispatchChunk + tid;
    const bool valid = a < n_assign;
    const int lr = valid ? inv[a] : -1;
    const int id = lr >= 0 ? ids[a] : 0;
    const int G = (kDispatchChunk / E) > 0 ? (kDispatchChunk / E) : 1;
    const int bpg = (nb + G - 1) / G;
    const int e = tid % E, g = tid / E;
    if (tid < E * G) {
        const int b0 = g * bpg, b1 = min(nb, b0 + bpg);
        int s_all = 0, s_bef = 0;
        for (int c0 = b0; c0 < b1; c0 += 8) {  // 8 independent loads in flight
            int c[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) c[u] = (c0 + u < b1) ? partial[(long)(c0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                s_all += c[u];
                s_bef += (c0 + u < b) ? c[u] : 0;
            }
        }
        gall[g * E + e] = s_all;
        gbef[g * E + e] = s_bef;
    }
    __syncthreads();
    int v = 0, bef = 0;
    if (tid < E)
        for (int i = 0; i < G; ++i) {
            v += gall[i * E + tid];
            bef += gbef[i * E + tid];
        }
    const int incl = wave_incl_scan(v);
    if (l == kWave - 1) wsum[wv] = incl;
    __syncthreads();
    int wbase = 0;
    for (int i = 0; i < wv; ++i) wbase += wsum[i];
    const int excl = wbase + incl - v;
    if (tid < E) {
        base[tid] = excl + bef;
        if (b == 0) {
            offsets[tid] = excl;
            if (tid == E - 1) offsets[E] = excl + v;
        }
    }
    __syncthreads();
    if (lr >= 0) {
        const int r = base[id] + lr;
        row_token[r] = a / k;
        inv[a] = r;
    }
}

// Token-major row copy: each wave takes TPW tokens, reads each token row of
// x once (all TPW rows' loads in flight before any store) and writes it to
// the k destination rows its assignments got (inv; dropped slots: none), so x
// is read T*H*b bytes once instead of once per assignment. The x loads are
// non-temporal (read once; prefill copy 52 -> 45 us); the stores are not,
// since the W1 launch reads x_perm right after.
template <int TPW, int VPL>
__global__ __launch_bounds__(256) void scatter_rows_kernel(const u32x4* __restrict__ x, const int32_t* __restrict__ inv,
                                                           int T, int k, int V, u32x4* __restrict__ out) {
    const int wave = threadIdx.x / kWave, l = lane_id();
    const long t0 = ((long)blockIdx.x * 4 + wave) * TPW;
    if (t0 >= T) return;
    for (int c0 = 0; c0 < V; c0 += kWave * VPL) {
        u32x4 v[TPW][VPL];
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int u = 0; u < VPL; ++u) {
                const int c = c0 + u * kWave + l;
                if (t0 + i < T && c < V) v[i][u] = __builtin_nontemporal_load(&x[(t0 + i) * V + c]);
            }
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            if (t0 + i >= T) break;
            for (int j = 0; j < k; ++j) {
                const int r = inv[(t0 + i) * k + j];  // wave-uniform
                if (r < 0) continue;
#pragma unroll
                for (int u = 0; u < VPL; ++u) {
                    const int c = c0 + u * kWave + l;
                    if (c < V) out[(long)r * V + c] = v[i][u];
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_count(const int32_t* ids, const float* w, int n_assign, int E, int32_t* partial, hipStream_t s) {
    const int nb = dispatch_blocks(n_assign);
    hipLaunchKernelGGL(count_kernel, dim3(nb), dim3(kDispatchChunk), 0, s, ids, w, n_assign, E, partial);
    return hipGetLastError();
}

hipError_t launch_dispatch_small(const int32_t* ids, const float* w, int n_assign, int k, int E, int32_t* offsets,
                                 int32_t* row_token, int32_t* inv, hipStream_t s) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(kSmallAssign), 0, s, ids, w, n_assign, k, E,
                       expert_bits(E), offsets, row_token, inv);
    return hipGetLastError();
}

bool dispatch_two_pass(long n_assign, int E) { return (long)dispatch_blocks(n_assign) * E <= kFinalizeCounts; }

hipError_t launch_count_rank(const int32_t* ids, const float* w, int n_assign, int E, int32_t* partial, int32_t* inv,
                             hipStream_t s) {
    hipLaunchKernelGGL(count_rank_kernel, dim3(dispatch_blocks(n_assign)), dim3(kDispatchChunk), 0, s, ids, w,
                       n_assign, E, expert_bits(E), partial, inv);
    return hipGetLastError();
}

hipError_t launch_finalize(const int32_t* ids, const int32_t* partial, int n_assign, int k, int E, int32_t* offsets,
                           int32_t* row_token, int32_t* inv, hipStream_t s) {
    const int nb = dispatch_blocks(n_assign);
    hipLaunchKernelGGL(finalize_kernel, dim3(nb), dim3(kDispatchChunk), 0, s, ids, partial, nb, n_assign, k, E,
                       offsets, row_token, inv);
    return hipGetLastError();
}

hipError_t launch_scan(int32_t* partial, int n_blocks, int E, int32_t* offsets, hipStream_t s) {
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, partial, n_blocks, E, offsets);
    return hipGetLastError();
}

hipError_t launch_index(const int32_t* ids, const float* w, const int32_t* partial, int n_assign, int k, int E,
                        int32_t* row_token, int32_t* inv, hipStream_t s) {
    const int nb = dispatch_blocks(n_assign);
    hipLaunchKernelGGL(index_kernel, dim3(nb), dim3(kDispatchChunk), 0, s, ids, w, partial, n_assign, k, E, expert_bits(E),
                       row_token, inv);
    return hipGetLastError();
}

hipError_t launch_copy_rows(const void* x, const int32_t* inv, int T, int k, int row_bytes, void* x_perm,
                            hipStream_t s) {
    const int V = row_bytes / 16;
    if (T == 0) return hipSuccess;
    if (T >= 4096) {  // 16 loads of 16 bytes in flight per lane
        hipLaunchKernelGGL((scatter_rows_kernel<4, 4>), dim3((unsigned)((T + 15) / 16)), dim3(256), 0, s,
                           (const u32x4*)x, inv, T, k, V, (u32x4*)x_perm);
    } else {  // few tokens: one per wave, for more workgroups
        hipLaunchKernelGGL((scatter_rows_kernel<1, 4>), dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s,
                           (const u32x4*)x, inv, T, k, V, (u32x4*)x_perm);
    }
    return hipGetLastError();
}

}  // namespace moe

// ---------------------------------------------------------------------------
// Padded fixed-shape layout (the ablation of the ragged scheduler): every
// expert gets exactly C rows. Page 3, section "单机MoE执行流水线": batching
// experts with different row counts either pads them to one shape or runs a
// grouped kernel over the ragged groups; this is the padded alternative.
namespace moe {

namespace {

// x_pad[e*C + i] = x[row_token[offsets[e] + i]] for i < count_e (and i < C),
// zero for the padding rows. One wave per padded row, 16-byte chunks.
__global__ __launch_bounds__(256) void pad_rows_kernel(const u32x4* __restrict__ x, const int32_t* __restrict__ row_token,
                                                       const int32_t* __restrict__ offsets, int C, long rows, int V,
                                                       u32x4* __restrict__ x_pad) {
    const long p = (long)blockIdx.x * 4 + threadIdx.x / kWave;
    if (p >= rows) return;
    const int e = (int)(p / C), i = (int)(p % C);
    const int cnt = offsets[e + 1] - offsets[e];
    const long src = i < cnt ? (long)row_token[offsets[e] + i] * V : -1;
    for (int c = lane_id(); c < V; c += kWave) x_pad[p * V + c] = src >= 0 ? x[src + c] : u32x4{0u, 0u, 0u, 0u};
}

// inv_pad[t*k+j] = e*C + (inv - offsets[e]) for a kept slot whose row index
// inside its expert is < C, else -1 (dropped, or beyond the padded shape).
__global__ __launch_bounds__(256) void pad_inv_kernel(const int32_t* __restrict__ ids, const int32_t* __restrict__ inv,
                                                      const int32_t* __restrict__ offsets, long n, int E, int C,
                                                      int32_t* __restrict__ inv_pad) {
    const long a = (long)blockIdx.x * 256 + threadIdx.x;
    if (a >= n) return;
    const int r = inv[a], e = ids[a];
    int out = -1;
    if (r >= 0 && (unsigned)e < (unsigned)E) {
        const int i = r - offsets[e];
        if (i < C) out = e * C + i;
    }
    inv_pad[a] = out;
}

__global__ void uniform_offsets_kernel(int32_t* __restrict__ offsets, int E, int C) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e <= E) offsets[e] = e * C;
}

}  // namespace

hipError_t launch_pad_dispatch(const void* x, const int32_t* ids, const int32_t* offsets, const int32_t* row_token,
                               const int32_t* inv, int T, int k, int E, int C, int row_bytes, void* x_pad,
                               int32_t* inv_pad, hipStream_t s) {
    const long rows = (long)E * C;
    const int V = row_bytes / 16;
    if (rows > 0)
        hipLaunchKernelGGL(pad_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, (const u32x4*)x,
                           row_token, offsets, C, rows, V, (u32x4*)x_pad);
    const long n = (long)T * k;
    hipLaunchKernelGGL(pad_inv_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ids, inv, offsets, n, E, C,
                       inv_pad);
    return hipGetLastError();
}

hipError_t launch_uniform_offsets(int32_t* offsets, int E, int C, hipStream_t s) {
    hipLaunchKernelGGL(uniform_offsets_kernel, dim3((E + 1 + 255) / 256), dim3(256), 0, s, offsets, E, C);
    return hipGetLastError();
}

}  // namespace moe
