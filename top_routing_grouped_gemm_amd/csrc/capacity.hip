// Capacity-limited top-k selection.
//
// Page 1 ("MoE大模型的智能调度…", www.jsqmd.com/news/1091713), section 3.2,
// second routing pitfall: every expert accepts at most
// capacity = tokens * k / experts * 1.2 selections; an expert chosen more
// often has its logit set to -inf for the excess tokens, which choose again.
// Tokens have priority by ascending id, so the result is the one where token
// t takes its k best experts among those the tokens before it have not yet
// filled (ties to the lower expert id).
//
// That definition is sequential over tokens. It is reached here in parallel
// rounds on a per-expert cut-off tau[e] (expert e is available to tokens
// t < tau[e]): start with tau = T; a round selects every token's top-k among
// its available experts, then sets tau[e] to one past the token holding e's
// cap-th selection (when e has that many). tau only decreases, a token's
// choice among a shrinking set keeps every expert it still can, and the
// unique fixed point is the sequential result (an expert with cap holders up
// to token t* is full for every later token). One launch per round: every
// workgroup selects a chunk of tokens and histograms it; the last workgroup
// to finish (device-scope counter, release/acquire fences) tightens tau and
// raises a done flag when nothing moved; later launches then return at once.
// If kCapMaxRounds rounds do not converge, a one-wave kernel runs the
// sequential definition itself, so the result is exact either way. A last
// kernel computes the softmax weights (and drop) over each token's final
// selection. No count ever returns to the host.
#include "moe_internal.hpp"
#include "topk.hpp"

namespace moe {

namespace {

constexpr int kCapThreads = 1024;                // 16 waves per round workgroup
constexpr int kCapWaves = kCapThreads / kWave;
constexpr int kCapTPW = 4;                       // tokens per wave, logit rows loaded up front
constexpr int kCapChunk = kCapWaves * kCapTPW;   // 64 tokens per workgroup
static_assert(kCapChunk == kWave, "the holder search gives one lane per token of a chunk");
constexpr int kCapMaxE = 1024;
enum { kDone = 0, kCounter = 1, kRounds = 2 };

struct CapWs {
    int* tau;   // [E]
    int* ctl;   // [4]: done flag, arrival counter, rounds run
    int* hist;  // [nchunks][E]
};

inline int cap_chunks(int T) { return (T + kCapChunk - 1) / kCapChunk; }

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

CapWs cap_ws(void* ws, int E) {
    char* b = (char*)ws;
    CapWs w;
    w.tau = (int*)b;
    w.ctl = (int*)(b + align256((size_t)E * 4));
    w.hist = (int*)(b + align256((size_t)E * 4) + 256);
    return w;
}

__global__ void cap_init_kernel(int* __restrict__ tau, int* __restrict__ ctl, int E, int T) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < E) tau[i] = T;
    if (i < 4) ctl[i] = 0;
}

// Keys of one token's experts: available ones keyed by logit, others 0.
template <int Q>
__device__ __forceinline__ void token_keys(const float* __restrict__ row, int E, long t, const int* avail_until,
                                           float (&v)[Q], uint32_t (&key)[Q]) {
    const int l = lane_id();
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int e = q * kWave + l;
        v[q] = e < E ? row[e] : -INFINITY;
        key[q] = (e < E && t < avail_until[e]) ? ord_key(v[q] + 0.0f) : 0u;
    }
}

template <int Q>
__global__ __launch_bounds__(kCapThreads) void cap_round_kernel(const float* __restrict__ logits, int ld, int T, int E,
                                                                int k, int cap, int* __restrict__ tau,
                                                                int* __restrict__ ctl, int* __restrict__ hist,
                                                                int32_t* __restrict__ ids, int nchunks) {
    __shared__ int tau_s[kCapMaxE];
    __shared__ int h[kCapMaxE];    // chunk histogram, then per-group sums [G][E]
    __shared__ int cross[kCapMaxE];  // chunk * 64 + rank - 1 of the cap-th holder, or -1
    __shared__ int last, changed;
    if (__hip_atomic_load(&ctl[kDone], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;  // converged
    const int tid = threadIdx.x, wave = tid / kWave, l = lane_id();
    const long t0 = (long)blockIdx.x * kCapChunk + wave * kCapTPW;
    float v[kCapTPW][Q];  // this wave's token rows, all loads issued before any selection
#pragma unroll
    for (int i = 0; i < kCapTPW; ++i)
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int e = q * kWave + l;
            v[i][q] = (t0 + i < T && e < E) ? logits[(t0 + i) * ld + e] : -INFINITY;
        }
    for (int e = tid; e < E; e += kCapThreads) {
        tau_s[e] = tau[e];
        h[e] = 0;
    }
    if (tid == 0) changed = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kCapTPW; ++i) {
        const long t = t0 + i;
        if (t >= T) break;  // wave-uniform
        uint32_t key[Q];
        bool sel[Q], kept[Q];
        float p[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int e = q * kWave + l;
            key[q] = (e < E && t < tau_s[e]) ? ord_key(v[i][q] + 0.0f) : 0u;
            kept[q] = false;
            p[q] = 0.0f;
        }
        radix_select<Q, true>(key, k, sel);
        write_slots<Q>(sel, kept, p, t, k, ids, nullptr);
#pragma unroll
        for (int q = 0; q < Q; ++q)
            if (sel[q]) atomicAdd(&h[q * kWave + l], 1);  // order-free: only a count
    }
    __syncthreads();
    for (int e = tid; e < E; e += kCapThreads) hist[(long)blockIdx.x * E + e] = h[e];
    // The barrier completes every wave's stores of this workgroup; one thread's
    // device-scope fences then act on the shared caches for all of them: the
    // release writes this XCD's L2 back so the other XCDs see the ids and the
    // histogram, the acquire in the last workgroup drops stale cached lines
    // before it reads everybody's results.
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        last = __hip_atomic_fetch_add(&ctl[kCounter], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == nchunks - 1;
        if (last) __threadfence();
    }
    __syncthreads();
    if (!last) return;

    // Last workgroup. (1) Where does expert e's count reach cap? G groups of E
    // threads each sum a contiguous range of chunks (16 loads in flight), the
    // group whose range holds the crossing finds the chunk and the rank there.
    const int G = kCapThreads / E > 0 ? kCapThreads / E : 1;
    const int per = (nchunks + G - 1) / G;
    const int g = tid / E, e = tid % E;
    const bool act = g < G && tid < G * E;
    const int c_lo = g * per, c_hi = min(nchunks, c_lo + per);
    int gs = 0;
    if (act) {
        for (int c0 = c_lo; c0 < c_hi; c0 += 16) {
            int hc[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) hc[u] = c0 + u < c_hi ? hist[(long)(c0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 16; ++u) gs += hc[u];
        }
    }
    __syncthreads();  // h becomes the [G][E] group sums
    if (act) h[g * E + e] = gs;
    for (int x = tid; x < E; x += kCapThreads) cross[x] = -1;
    __syncthreads();
    if (act) {
        int base = 0;
        for (int i = 0; i < g; ++i) base += h[i * E + e];
        if (base < cap && base + gs >= cap) {  // the cap-th holder is in this group's range
            int run = base;
            for (int c = c_lo; c < c_hi; ++c) {
                const int hc = hist[(long)c * E + e];
                if (run + hc >= cap) {
                    cross[e] = c * kCapChunk + (cap - run) - 1;
                    break;
                }
                run += hc;
            }
        }
    }
    __syncthreads();
    // (2) The holder itself: one wave per crossing expert, lane i tests token
    // chunk*64 + i; the (rank)-th set bit of the ballot, in token order.
    for (int x = wave; x < E; x += kCapWaves) {
        const int cr = cross[x];
        if (cr < 0) continue;  // wave-uniform (LDS value)
        const int c = cr / kCapChunk, rank = cr % kCapChunk;  // rank: 0-based
        const long t = (long)c * kCapChunk + l;
        bool has = false;
        if (t < T)
            for (int j = 0; j < k; ++j) has = has || ids[t * k + j] == x;
        unsigned long long m = __ballot(has);
        for (int i = 0; i < rank; ++i) m &= m - 1;  // drop the lowest set bits before the wanted one
        const int tnew = c * kCapChunk + __ffsll((long long)m) - 1 + 1;
        if (l == 0 && tnew < tau_s[x]) {
            tau[x] = tnew;
            atomicOr(&changed, 1);
        }
    }
    __syncthreads();
    if (tid == 0) {
        if (!changed) ctl[kDone] = 1;
        ctl[kCounter] = 0;
        ctl[kRounds] += 1;
    }
}

// The sequential definition itself (one wave), run only if the rounds did not
// converge: token by token, experts with cap selections are unavailable.
template <int Q>
__global__ __launch_bounds__(64) void cap_serial_kernel(const float* __restrict__ logits, int ld, int T, int E, int k,
                                                        int cap, const int* __restrict__ ctl,
                                                        int32_t* __restrict__ ids) {
    __shared__ int until[kCapMaxE];  // T while the expert has room, else 0
    __shared__ int cnt[kCapMaxE];
    if (ctl[kDone] != 0) return;
    const int l = lane_id();
    for (int e = l; e < E; e += kWave) {
        until[e] = T;
        cnt[e] = 0;
    }
    __syncthreads();
    for (long t = 0; t < T; ++t) {
        float v[Q];
        uint32_t key[Q];
        bool sel[Q], kept[Q];
        float p[Q];
        token_keys<Q>(logits + t * ld, E, t, until, v, key);
        radix_select<Q, true>(key, k, sel);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            kept[q] = sel[q];
            p[q] = 0.0f;
        }
        write_slots<Q>(sel, kept, p, t, k, ids, nullptr);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int e = q * kWave + l;
            if (sel[q] && ++cnt[e] >= cap) until[e] = 0;  // each expert belongs to one lane
        }
        __syncthreads();
    }
}

// Softmax weights over each token's final selection, optional drop.
template <int Q>
__global__ __launch_bounds__(256) void cap_weights_kernel(const float* __restrict__ logits, int ld, int T, int E,
                                                          int k, float drop, int32_t* __restrict__ ids,
                                                          float* __restrict__ wout) {
    const long t = (long)blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    const int l = lane_id();
    float v[Q], p[Q];
    bool sel[Q], kept[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int e = q * kWave + l;
        v[q] = e < E ? logits[t * ld + e] : -INFINITY;
        sel[q] = false;
    }
    for (int j = 0; j < k; ++j) {
        const int id = ids[t * k + j];
#pragma unroll
        for (int q = 0; q < Q; ++q) sel[q] = sel[q] || (q * kWave + l == id);
    }
    softmax_drop<Q>(v, sel, drop, p, kept);
    write_slots<Q>(sel, kept, p, t, k, ids, wout);
}

template <int Q>
hipError_t run_capacity(const float* logits, int ld, int T, int E, int k, int cap, float drop, int32_t* ids,
                        float* w, void* ws, hipStream_t s) {
    const CapWs c = cap_ws(ws, E);
    const int nchunks = cap_chunks(T);
    hipLaunchKernelGGL(cap_init_kernel, dim3((E + 255) / 256), dim3(256), 0, s, c.tau, c.ctl, E, T);
    for (int r = 0; r < kCapMaxRounds; ++r)
        hipLaunchKernelGGL((cap_round_kernel<Q>), dim3(nchunks), dim3(kCapThreads), 0, s, logits, ld, T, E, k, cap,
                           c.tau, c.ctl, c.hist, ids, nchunks);
    hipLaunchKernelGGL((cap_serial_kernel<Q>), dim3(1), dim3(64), 0, s, logits, ld, T, E, k, cap,
                       (const int*)c.ctl, ids);
    hipLaunchKernelGGL((cap_weights_kernel<Q>), dim3((T + 3) / 4), dim3(256), 0, s, logits, ld, T, E, k, drop, ids,
                       w);
    return hipGetLastError();
}

}  // namespace

size_t capacity_workspace_bytes(int T, int E) {
    return align256((size_t)E * 4) + 256 + align256((size_t)cap_chunks(T) * E * 4);
}

hipError_t launch_capacity_select(const float* logits, int ld, int T, int E, int k, int cap, float drop,
                                  int32_t* ids, float* w, void* ws, hipStream_t s) {
    if (E <= kWave) return run_capacity<1>(logits, ld, T, E, k, cap, drop, ids, w, ws, s);
    if (E <= 2 * kWave) return run_capacity<2>(logits, ld, T, E, k, cap, drop, ids, w, ws, s);
    if (E <= 4 * kWave) return run_capacity<4>(logits, ld, T, E, k, cap, drop, ids, w, ws, s);
    if (E <= 8 * kWave) return run_capacity<8>(logits, ld, T, E, k, cap, drop, ids, w, ws, s);
    return run_capacity<16>(logits, ld, T, E, k, cap, drop, ids, w, ws, s);
}

}  // namespace moe
