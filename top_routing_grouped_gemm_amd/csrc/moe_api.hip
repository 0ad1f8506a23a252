// C ABI of the MoE-layer forward (declared in include/moe.h): argument
// checks, workspace layout and the launch sequence on the caller's stream.
#include <math.h>

#include <mutex>

#include "moe.h"

#include "moe_internal.hpp"

namespace {

using moe::Dtype;

constexpr size_t kAlign = 256;
constexpr int kMaxExperts = 1024;
constexpr int kMaxK = 32;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t elem_bytes(moe_dtype_t dt) { return dt == MOE_BF16 ? 2 : 4; }

bool valid_dtype(moe_dtype_t dt) { return dt == MOE_F32 || dt == MOE_BF16; }

// Size checks shared by all entry points; F == 0 / Fs < 0 skip the checks that
// do not apply to a call.
int check_sizes(int T, int H, int F, int E, int k) {
    if (T < 1 || H < 1 || E < 1 || k < 1 || k > E || F < 0) return MOE_ERR_INVALID_ARG;
    if (E > kMaxExperts || k > kMaxK) return MOE_ERR_UNSUPPORTED;
    if (H % 8 != 0 || F % 8 != 0) return MOE_ERR_UNSUPPORTED;
    if ((long long)T * k >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int check_drop(float drop, int k) {
    if (!(drop >= 0.0f)) return MOE_ERR_INVALID_ARG;  // also rejects NaN
    if ((double)drop > (1.0 / (double)k) * (1.0 + 1e-6)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

struct FfnLayout {
    size_t h, h_sh, total;
};

FfnLayout ffn_layout(int T, int F, int k, int Fs, moe_dtype_t dt) {
    FfnLayout L;
    size_t off = 0;
    L.h = off;
    off = align_up(off + (size_t)T * k * F * elem_bytes(dt));
    L.h_sh = off;
    if (Fs > 0) off = align_up(off + (size_t)T * Fs * elem_bytes(dt));
    L.total = off;
    return L;
}

size_t permute_bytes(int T, int E, int k) {
    return align_up((size_t)moe::dispatch_blocks((long)T * k) * E * sizeof(int32_t));
}

struct FwdLayout {
    size_t ids, w, offsets, inv, row_token, partial, x_perm, y_perm, y_sh, ffn, route, total;
};

FwdLayout fwd_layout(int T, int H, int F, int E, int k, int Fs, moe_dtype_t dt) {
    FwdLayout L;
    const size_t TK = (size_t)T * k;
    size_t off = 0;
    L.ids = off;
    off = align_up(off + TK * sizeof(int32_t));
    L.w = off;
    off = align_up(off + TK * sizeof(float));
    L.offsets = off;
    off = align_up(off + (size_t)(E + 1) * sizeof(int32_t));
    L.inv = off;
    off = align_up(off + TK * sizeof(int32_t));
    L.row_token = off;
    off = align_up(off + TK * sizeof(int32_t));
    L.partial = off;
    off = align_up(off + permute_bytes(T, E, k));
    L.x_perm = off;
    off = align_up(off + TK * H * elem_bytes(dt));
    L.y_perm = off;
    off = align_up(off + TK * H * sizeof(float));
    L.y_sh = off;
    if (Fs > 0) off = align_up(off + (size_t)T * H * sizeof(float));
    L.ffn = off;
    off = align_up(off + ffn_layout(T, F, k, Fs, dt).total);
    L.route = off;
    off = align_up(off + moe::route_workspace_bytes(T, H, E, (Dtype)dt));
    L.total = off;
    return L;
}

// Workspace of moe_forward_mxfp8: routing and dispatch maps as in moe_forward,
// the MX codes and scales of x and of the SiLU output, and y_perm in block-scaled fp16.
struct MxLayout {
    size_t ids, w, offsets, inv, row_token, partial, route, xq, xs, hq, hs, y, total;
};

MxLayout mx_layout(int T, int H, int F, int E, int k) {
    MxLayout L;
    const size_t TK = (size_t)T * k;
    size_t off = 0;
    auto take = [&](size_t& field, size_t bytes) {
        field = off;
        off = align_up(off + bytes);
    };
    take(L.ids, TK * sizeof(int32_t));
    take(L.w, TK * sizeof(float));
    take(L.offsets, (size_t)(E + 1) * sizeof(int32_t));
    take(L.inv, TK * sizeof(int32_t));
    take(L.row_token, TK * sizeof(int32_t));
    take(L.partial, permute_bytes(T, E, k));
    take(L.route, moe::route_workspace_bytes(T, H, E, moe::kBF16));
    take(L.xq, (size_t)T * H);
    take(L.xs, (size_t)(H / 128) * T * 4);
    take(L.hq, TK * F);
    take(L.hs, (size_t)(F / 128) * TK * 4);
    take(L.y, TK * H * 2 + TK * (H / 32));
    L.total = off;
    return L;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                          \
    do {                                       \
        hipError_t _e = (expr);                \
        if (_e != hipSuccess) return MOE_ERR_HIP; \
    } while (0)

// copy_rows = false: only the routing maps (offsets, row_token, inv) are
// built and x_perm is left unwritten (the W1 launch then gathers x rows).
int enqueue_permute(const void* x, const int32_t* ids, const float* w, int T, int H, int E, int k,
                    moe_dtype_t dt, void* x_perm, int32_t* offsets, int32_t* row_token, int32_t* inv,
                    int32_t* partial, bool copy_rows, hipStream_t s) {
    const int n = T * k;
    if (n <= moe::kSmallAssign) {
        MOE_TRY(moe::launch_dispatch_small(ids, w, n, k, E, offsets, row_token, inv, s));
    } else if (moe::dispatch_two_pass(n, E)) {
        MOE_TRY(moe::launch_count_rank(ids, w, n, E, partial, inv, s));
        MOE_TRY(moe::launch_finalize(ids, partial, n, k, E, offsets, row_token, inv, s));
    } else {
        MOE_TRY(moe::launch_count(ids, w, n, E, partial, s));
        MOE_TRY(moe::launch_scan(partial, moe::dispatch_blocks(n), E, offsets, s));
        MOE_TRY(moe::launch_index(ids, w, partial, n, k, E, row_token, inv, s));
    }
    if (copy_rows) MOE_TRY(moe::launch_copy_rows(x, inv, T, k, (int)(H * elem_bytes(dt)), x_perm, s));
    return MOE_OK;
}

// Router, then the dispatch maps (+ the row copy when copy_rows).
int enqueue_route_permute(const void* x, const void* Wr, const float* bias, int T, int H, int E, int k, float drop,
                          moe_dtype_t dt, int32_t* ids, float* w, void* route_ws, void* x_perm, int32_t* offsets,
                          int32_t* row_token, int32_t* inv, int32_t* partial, bool copy_rows, hipStream_t s) {
    MOE_TRY(moe::launch_route(x, Wr, bias, T, H, E, k, drop, (Dtype)dt, ids, w, route_ws, s));
    return enqueue_permute(x, ids, w, T, H, E, k, dt, x_perm, offsets, row_token, inv, partial, copy_rows, s);
}

// row_token != NULL: the W1 launch gathers rows of x through row_token instead of reading x_perm.
// packed: y_perm is written in the block-scaled fp16 form of ffn_down_packs (the caller checked that it applies).
int enqueue_ffn(const void* x_perm, const int32_t* row_token, const int32_t* offsets, const void* W1, const void* W2,
                int T, int H, int F, int E, int k, moe_dtype_t dt, float* y_perm, const void* x, const void* W1s,
                const void* W2s, int Fs, float* y_shared, void* ws, bool packed, hipStream_t s) {
    const FfnLayout L = ffn_layout(T, F, k, Fs, dt);
    char* base = (char*)ws;
    void* h = base + L.h;
    const Dtype d = (Dtype)dt;
    const int rows = T * k;
    const moe::TileCfg cfg = moe::choose_tile(rows, E);
    const long hc = moe::h_blocked(cfg, H, F, rows, d);  // h layout shared by the W1 and W2 launches
    // shared expert: every token, read from x directly. Where the routed launches' tile shape allows it
    // (page 3, "MoE层的结构与token路由": the shared expert sees every token besides the routed ones), it is one
    // more group of T rows in the same two launches; otherwise two launches of its own.
    void* hs = base + L.h_sh;
    const bool merged = W1s != nullptr && moe::ffn_shared_merges(cfg, H, F, Fs, d);
    const moe::TileCfg cs = merged ? moe::kTileM128 : moe::choose_tile(T, 1);
    const long hsc = W1s != nullptr ? moe::h_blocked(cs, H, Fs, T, d) : 0;
    const moe::SharedGroup sg{x, W1s, W2s, hs, hsc, y_shared, T};
    const moe::SharedGroup* sh = merged ? &sg : nullptr;
    if (row_token != nullptr)
        MOE_TRY(moe::launch_ffn_up_gather(x, row_token, offsets, E, rows, W1, H, F, cfg, hc, h, s, sh));
    else
        MOE_TRY(moe::launch_ffn_up(x_perm, offsets, E, 0, rows, W1, H, F, d, h, cfg, hc, s, sh));
    if (W1s != nullptr && !merged) MOE_TRY(moe::launch_ffn_up(x, nullptr, 1, T, T, W1s, H, Fs, d, hs, cs, hsc, s));
    if (packed)
        MOE_TRY(moe::launch_ffn_down_packed(h, offsets, E, rows, W2, F, H, cfg, hc, y_perm, rows, s, sh));
    else
        MOE_TRY(moe::launch_ffn_down(h, offsets, E, 0, rows, W2, F, H, d, y_perm, cfg, hc, s, sh));
    if (W1s != nullptr && !merged)
        MOE_TRY(moe::launch_ffn_down(hs, nullptr, 1, T, T, W2s, Fs, H, d, y_shared, cs, hsc, s));
    return MOE_OK;
}

// Device buffers of one forward pass (inside a caller workspace or the no-allocation scratch array).
struct FwdBuffers {
    int32_t *ids, *off, *inv, *row_token, *partial;
    float *w, *y_perm, *y_sh;
    void *x_perm, *ffn, *route;
};

int check_forward(const void* x, const void* Wr, const void* W1, const void* W2, const void* W1s, const void* W2s,
                  int Fs, int T, int H, int F, int E, int k, float drop_thresh, moe_dtype_t dt, const void* y,
                  moe_dtype_t out_dt) {
    if (!valid_dtype(dt) || !valid_dtype(out_dt)) return MOE_ERR_INVALID_ARG;
    if (F < 1) return MOE_ERR_INVALID_ARG;
    int st = check_sizes(T, H, F, E, k);
    if (st != MOE_OK) return st;
    if ((st = check_drop(drop_thresh, k)) != MOE_OK) return st;
    if (!x || !Wr || !W1 || !W2 || !y) return MOE_ERR_INVALID_ARG;
    if ((W1s == nullptr) != (W2s == nullptr)) return MOE_ERR_INVALID_ARG;
    if (W1s != nullptr) {
        if (Fs < 1) return MOE_ERR_INVALID_ARG;
        if (Fs % 8 != 0) return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}

// The launch sequence of moe_forward on the buffers in b (caller-given debug outputs replace their buffers).
int enqueue_forward(const void* x, const void* Wr, const float* bias, const void* W1, const void* W2,
                    const void* W1s, const void* W2s, int fs, int T, int H, int F, int E, int k, float drop_thresh,
                    moe_dtype_t dt, void* y, moe_dtype_t out_dt, int32_t* topk_ids, float* topk_w,
                    int32_t* expert_offsets, int32_t* inv, const FwdBuffers& b, hipStream_t stream) {
    int32_t* ids = topk_ids ? topk_ids : b.ids;
    float* w = topk_w ? topk_w : b.w;
    int32_t* off = expert_offsets ? expert_offsets : b.off;
    int32_t* iv = inv ? inv : b.inv;
    // direct-to-LDS shapes: the W1 launch gathers x rows itself (x_perm is never written) and the W2 launch
    // writes y_perm as block-scaled fp16 (the combine reads 2 + 1/32 bytes per value instead of 4)
    const moe::TileCfg cfg = moe::choose_tile((long)T * k, E);
    const bool gather = moe::ffn_up_gathers(cfg, H, F, (Dtype)dt);
    const bool packed = moe::ffn_down_packs(cfg, F, H, (Dtype)dt);
    int st;
    if ((st = enqueue_route_permute(x, Wr, bias, T, H, E, k, drop_thresh, dt, ids, w, b.route, b.x_perm, off,
                                    b.row_token, iv, b.partial, !gather, stream)) != MOE_OK)
        return st;
    if ((st = enqueue_ffn(b.x_perm, gather ? b.row_token : nullptr, off, W1, W2, T, H, F, E, k, dt, b.y_perm, x, W1s,
                          W2s, fs, b.y_sh, b.ffn, packed, stream)) != MOE_OK)
        return st;
    if (packed)
        return hip_status(
            moe::launch_combine_packed(b.y_perm, (long)T * k, iv, w, b.y_sh, T, H, k, (Dtype)out_dt, y, stream));
    return hip_status(moe::launch_combine(b.y_perm, iv, w, b.y_sh, T, H, k, (Dtype)out_dt, y, stream));
}

// Layout of the no-allocation forward inside its scratch array: only the buffers the chosen kernels use
// (no x_perm when the W1 launch gathers rows of x; y_perm at 2 + 1/32 bytes per value when W2 packs it).
struct TightLayout {
    size_t ids, w, offsets, inv, row_token, partial, x_perm, y_perm, y_sh, ffn, route, total;
    bool gather;
};

TightLayout tight_layout(int T, int H, int F, int E, int k, int Fs, moe_dtype_t dt) {
    TightLayout L;
    const size_t TK = (size_t)T * k;
    const moe::TileCfg cfg = moe::choose_tile((long)TK, E);
    L.gather = moe::ffn_up_gathers(cfg, H, F, (Dtype)dt);
    const bool packed = moe::ffn_down_packs(cfg, F, H, (Dtype)dt);
    size_t off = 0;
    auto take = [&](size_t& field, size_t bytes) {
        field = off;
        off = align_up(off + bytes);
    };
    take(L.ids, TK * sizeof(int32_t));
    take(L.w, TK * sizeof(float));
    take(L.offsets, (size_t)(E + 1) * sizeof(int32_t));
    take(L.inv, TK * sizeof(int32_t));
    take(L.row_token, TK * sizeof(int32_t));
    take(L.partial, permute_bytes(T, E, k));
    take(L.x_perm, L.gather ? 0 : TK * H * elem_bytes(dt));
    take(L.y_perm, packed ? TK * H * 2 + TK * (H / 32) : TK * H * sizeof(float));
    take(L.y_sh, Fs > 0 ? (size_t)T * H * sizeof(float) : 0);
    take(L.ffn, ffn_layout(T, F, k, Fs, dt).total);
    take(L.route, moe::route_workspace_bytes(T, H, E, (Dtype)dt));
    L.total = off;
    return L;
}

int check_shared(const void* x, const void* W1s, const void* W2s, int Fs, const float* y_shared) {
    if (W1s == nullptr && W2s == nullptr) return MOE_OK;
    if (W1s == nullptr || W2s == nullptr || x == nullptr || y_shared == nullptr) return MOE_ERR_INVALID_ARG;
    if (Fs < 1) return MOE_ERR_INVALID_ARG;
    if (Fs % 8 != 0) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

}  // namespace

// Scratch memory of moe_forward_noalloc, for callers that cannot allocate: one array per GPU that the library
// runs on, held until the process ends. In host code `scratch` only names the symbol; its device address comes
// from hipGetSymbolAddress, once per device, and only that address is ever passed to a kernel.
constexpr size_t kNoAllocScratchBytes = 64u << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that `stream` belongs to (the current device for the null stream).
hipError_t scratch_address(hipStream_t stream, char** out) {
    int dev = -1;
    hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = (char*)p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

const char* moe_strerror(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: a size, pointer, threshold or dtype is invalid";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: sizes outside the supported limits";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than required";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: a kernel launch failed";
        default: return "unknown moe status";
    }
}

const char* moe_version(void) { return "0.1.0"; }

size_t moe_route_workspace_bytes(int T, int H, int E, moe_dtype_t dt) {
    if (!valid_dtype(dt) || check_sizes(T, H, 0, E, 1) != MOE_OK) return 0;
    return moe::route_workspace_bytes(T, H, E, (Dtype)dt);
}

size_t moe_permute_workspace_bytes(int T, int E, int k) {
    if (check_sizes(T, 8, 0, E, k) != MOE_OK) return 0;
    return permute_bytes(T, E, k);
}

size_t moe_ffn_workspace_bytes(int T, int F, int E, int k, int Fs, moe_dtype_t dt) {
    if (!valid_dtype(dt) || check_sizes(T, 8, F, E, k) != MOE_OK || F < 1 || Fs < 0 || Fs % 8 != 0) return 0;
    return ffn_layout(T, F, k, Fs, dt).total;
}

size_t moe_workspace_bytes(int T, int H, int F, int E, int k, int Fs, moe_dtype_t dt) {
    if (!valid_dtype(dt) || check_sizes(T, H, F, E, k) != MOE_OK || F < 1 || Fs < 0 || Fs % 8 != 0) return 0;
    return fwd_layout(T, H, F, E, k, Fs, dt).total;
}

int moe_route(const void* x, const void* Wr, const float* bias, int T, int H, int E, int k, float drop_thresh,
              moe_dtype_t dt, int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!valid_dtype(dt)) return MOE_ERR_INVALID_ARG;
    int st = check_sizes(T, H, 0, E, k);
    if (st != MOE_OK) return st;
    if ((st = check_drop(drop_thresh, k)) != MOE_OK) return st;
    if (!x || !Wr || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
    const size_t need = moe::route_workspace_bytes(T, H, E, (Dtype)dt);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return MOE_ERR_WORKSPACE;
    return hip_status(
        moe::launch_route(x, Wr, bias, T, H, E, k, drop_thresh, (Dtype)dt, topk_ids, topk_w, ws, stream));
}

size_t moe_grouped_ffn_padded_workspace_bytes(int E, int C, int H, int F, moe_dtype_t dt) {
    if (!valid_dtype(dt) || E < 1 || E > kMaxExperts || C < 1 || check_sizes(1, H, F, E, 1) != MOE_OK || F < 1)
        return 0;
    if ((long long)E * C >= (1LL << 31)) return 0;
    return align_up((size_t)(E + 1) * sizeof(int32_t)) + ffn_layout(E * C, F, 1, 0, dt).total;
}

int moe_pad_dispatch(const void* x, const int32_t* topk_ids, const int32_t* expert_offsets, const int32_t* row_token,
                     const int32_t* inv, int T, int H, int E, int k, int C, moe_dtype_t dt, void* x_pad,
                     int32_t* inv_pad, hipStream_t stream) {
    if (!valid_dtype(dt)) return MOE_ERR_INVALID_ARG;
    int st = check_sizes(T, H, 0, E, k);
    if (st != MOE_OK) return st;
    if (C < 1) return MOE_ERR_INVALID_ARG;
    if ((long long)E * C >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
    if (!x || !topk_ids || !expert_offsets || !row_token || !inv || !x_pad || !inv_pad) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_pad_dispatch(x, topk_ids, expert_offsets, row_token, inv, T, k, E, C,
                                               (int)(H * elem_bytes(dt)), x_pad, inv_pad, stream));
}

int moe_grouped_ffn_padded(const void* x_pad, const void* W1, const void* W2, int E, int C, int H, int F,
                           moe_dtype_t dt, float* y_pad, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!valid_dtype(dt)) return MOE_ERR_INVALID_ARG;
    if (E < 1 || C < 1 || H < 1 || F < 1) return MOE_ERR_INVALID_ARG;
    int st = check_sizes(1, H, F, E, 1);
    if (st != MOE_OK) return st;
    if ((long long)E * C >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
    if (!x_pad || !W1 || !W2 || !y_pad) return MOE_ERR_INVALID_ARG;
    const size_t need = moe_grouped_ffn_padded_workspace_bytes(E, C, H, F, dt);
    if (ws == nullptr || ws_bytes < need) return MOE_ERR_WORKSPACE;
    int32_t* offsets = (int32_t*)ws;
    void* ffn_ws = (char*)ws + align_up((size_t)(E + 1) * sizeof(int32_t));
    MOE_TRY(moe::launch_uniform_offsets(offsets, E, C, stream));
    // the same grouped kernels, over E groups of exactly C rows
    return enqueue_ffn(x_pad, nullptr, offsets, W1, W2, E * C, H, F, E, 1, dt, y_pad, nullptr, nullptr, nullptr, 0,
                       nullptr, ffn_ws, false, stream);
}

static int capacity_args(int T, int E, int k, int cap) {
    if (cap < 1) return MOE_ERR_INVALID_ARG;
    if ((long long)E - ((long long)T * k) / cap < k) return MOE_ERR_UNSUPPORTED;  // some token could lack k experts
    return MOE_OK;
}

static size_t route_capacity_layout(int T, int H, int E, size_t* logits_off, size_t* sel_off) {
    const size_t part = align_up(moe::route_logits_partial_bytes(T, H, E));
    const size_t lg = align_up((size_t)T * moe::route_logits_ld(E) * sizeof(float));
    *logits_off = part;
    *sel_off = part + lg;
    return part + lg + align_up(moe::capacity_workspace_bytes(T, E));
}

size_t moe_select_capacity_workspace_bytes(int T, int E) {
    if (T < 1 || E < 1 || E > kMaxExperts) return 0;
    return align_up(moe::capacity_workspace_bytes(T, E));
}

size_t moe_route_capacity_workspace_bytes(int T, int H, int E, moe_dtype_t dt) {
    if (!valid_dtype(dt) || check_sizes(T, H, 0, E, 1) != MOE_OK) return 0;
    if (!moe::route_logits_ok(H, E, (Dtype)dt)) return 0;
    size_t a, b;
    return route_capacity_layout(T, H, E, &a, &b);
}

int moe_select_capacity(const float* logits, int T, int E, int k, float drop_thresh, int cap, int32_t* topk_ids,
                        float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_sizes(T, 8, 0, E, k);
    if (st != MOE_OK) return st;
    if ((st = check_drop(drop_thresh, k)) != MOE_OK) return st;
    if ((st = capacity_args(T, E, k, cap)) != MOE_OK) return st;
    if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
    if (ws == nullptr || ws_bytes < moe_select_capacity_workspace_bytes(T, E)) return MOE_ERR_WORKSPACE;
    return hip_status(
        moe::launch_capacity_select(logits, E, T, E, k, cap, drop_thresh, topk_ids, topk_w, ws, stream));
}

int moe_route_capacity(const void* x, const void* Wr, const float* bias, int T, int H, int E, int k,
                       float drop_thresh, double cap_factor, moe_dtype_t dt, int32_t* topk_ids, float* topk_w,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!valid_dtype(dt)) return MOE_ERR_INVALID_ARG;
    int st = check_sizes(T, H, 0, E, k);
    if (st != MOE_OK) return st;
    if ((st = check_drop(drop_thresh, k)) != MOE_OK) return st;
    if (!(cap_factor > 0.0) || !(cap_factor <= 1e6)) return MOE_ERR_INVALID_ARG;  // rejects NaN and inf
    const double capd = ceil((double)T * k / E * cap_factor);
    const int cap = capd >= 2147483647.0 ? 2147483647 : (int)capd;
    if ((st = capacity_args(T, E, k, cap)) != MOE_OK) return st;
    if (!x || !Wr || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
    if (!moe::route_logits_ok(H, E, (Dtype)dt)) return MOE_ERR_UNSUPPORTED;
    size_t lo, so;
    const size_t need = route_capacity_layout(T, H, E, &lo, &so);
    if (ws == nullptr || ws_bytes < need) return MOE_ERR_WORKSPACE;
    char* base = (char*)ws;
    float* logits = (float*)(base + lo);
    MOE_TRY(moe::launch_route_logits(x, Wr, bias, T, H, E, logits, base, stream));
    return hip_status(moe::launch_capacity_select(logits, moe::route_logits_ld(E), T, E, k, cap, drop_thresh,
                                                  topk_ids, topk_w, base + so, stream));
}

int moe_permute(const void* x, const int32_t* topk_ids, const float* topk_w, int T, int H, int E, int k,
                moe_dtype_t dt, void* x_perm, int32_t* expert_offsets, int32_t* row_token, int32_t* inv, void* ws,
                size_t ws_bytes, hipStream_t stream) {
    if (!valid_dtype(dt)) return MOE_ERR_INVALID_ARG;
    int st = check_sizes(T, H, 0, E, k);
    if (st != MOE_OK) return st;
    if (!x || !topk_ids || !topk_w || !x_perm || !expert_offsets || !row_token || !inv || !ws)
        return MOE_ERR_INVALID_ARG;
    if (ws_bytes < permute_bytes(T, E, k)) return MOE_ERR_WORKSPACE;
    return enqueue_permute(x, topk_ids, topk_w, T, H, E, k, dt, x_perm, expert_offsets, row_token, inv,
                           (int32_t*)ws, true, stream);
}

int moe_grouped_ffn(const void* x_perm, const int32_t* expert_offsets, const void* W1, const void* W2, int T, int H,
                    int F, int E, int k, moe_dtype_t dt, float* y_perm, const void* x, const void* W1s,
                    const void* W2s, int Fs, float* y_shared, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!valid_dtype(dt)) return MOE_ERR_INVALID_ARG;
    if (F < 1) return MOE_ERR_INVALID_ARG;
    int st = check_sizes(T, H, F, E, k);
    if (st != MOE_OK) return st;
    if ((st = check_shared(x, W1s, W2s, Fs, y_shared)) != MOE_OK) return st;
    if (!x_perm || !expert_offsets || !W1 || !W2 || !y_perm || !ws) return MOE_ERR_INVALID_ARG;
    const int fs = W1s ? Fs : 0;
    if (ws_bytes < ffn_layout(T, F, k, fs, dt).total) return MOE_ERR_WORKSPACE;
    return enqueue_ffn(x_perm, nullptr, expert_offsets, W1, W2, T, H, F, E, k, dt, y_perm, x, W1s, W2s, fs, y_shared,
                       ws, false, stream);
}

int moe_grouped_ffn_fused(const void* x_perm, const int32_t* expert_offsets, const void* W1, const void* W2, int T,
                          int H, int F, int E, int k, moe_dtype_t dt, float* y_perm, hipStream_t stream) {
    if (!valid_dtype(dt)) return MOE_ERR_INVALID_ARG;
    if (F < 1) return MOE_ERR_INVALID_ARG;
    const int st = check_sizes(T, H, F, E, k);
    if (st != MOE_OK) return st;
    if (!x_perm || !expert_offsets || !W1 || !W2 || !y_perm) return MOE_ERR_INVALID_ARG;
    if (!moe::ffn_fused_ok(H, F, (Dtype)dt)) return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_ffn_fused(x_perm, expert_offsets, E, T * k, W1, W2, H, F, y_perm, stream));
}

int moe_combine(const float* y_perm, const int32_t* inv, const float* topk_w, const float* y_shared, int T, int H,
                int k, moe_dtype_t out_dt, void* y, hipStream_t stream) {
    if (!valid_dtype(out_dt)) return MOE_ERR_INVALID_ARG;
    if (T < 1 || H < 1 || k < 1) return MOE_ERR_INVALID_ARG;
    if (H % 8 != 0 || k > kMaxK || (long long)T * k >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
    if (!y_perm || !inv || !topk_w || !y) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_combine(y_perm, inv, topk_w, y_shared, T, H, k, (Dtype)out_dt, y, stream));
}

int moe_forward(const void* x, const void* Wr, const float* bias, const void* W1, const void* W2, const void* W1s,
                const void* W2s, int Fs, int T, int H, int F, int E, int k, float drop_thresh, moe_dtype_t dt,
                void* y, moe_dtype_t out_dt, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                int32_t* inv, void* ws, size_t ws_bytes, hipStream_t stream) {
    const int st = check_forward(x, Wr, W1, W2, W1s, W2s, Fs, T, H, F, E, k, drop_thresh, dt, y, out_dt);
    if (st != MOE_OK) return st;
    if (!ws) return MOE_ERR_INVALID_ARG;
    const int fs = W1s ? Fs : 0;
    const FwdLayout L = fwd_layout(T, H, F, E, k, fs, dt);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    char* base = (char*)ws;
    FwdBuffers b;
    b.ids = (int32_t*)(base + L.ids);
    b.w = (float*)(base + L.w);
    b.off = (int32_t*)(base + L.offsets);
    b.inv = (int32_t*)(base + L.inv);
    b.row_token = (int32_t*)(base + L.row_token);
    b.partial = (int32_t*)(base + L.partial);
    b.x_perm = base + L.x_perm;
    b.y_perm = (float*)(base + L.y_perm);
    b.y_sh = fs > 0 ? (float*)(base + L.y_sh) : nullptr;
    b.ffn = base + L.ffn;
    b.route = base + L.route;
    return enqueue_forward(x, Wr, bias, W1, W2, W1s, W2s, fs, T, H, F, E, k, drop_thresh, dt, y, out_dt, topk_ids,
                           topk_w, expert_offsets, inv, b, stream);
}

int moe_forward_noalloc(const void* x, const void* Wr, const float* bias, const void* W1, const void* W2,
                        const void* W1s, const void* W2s, int Fs, int T, int H, int F, int E, int k,
                        float drop_thresh, moe_dtype_t dt, void* y, moe_dtype_t out_dt, int32_t* topk_ids,
                        float* topk_w, int32_t* expert_offsets, int32_t* inv, hipStream_t stream) {
    const int st = check_forward(x, Wr, W1, W2, W1s, W2s, Fs, T, H, F, E, k, drop_thresh, dt, y, out_dt);
    if (st != MOE_OK) return st;
    const int fs = W1s ? Fs : 0;
    const TightLayout L = tight_layout(T, H, F, E, k, fs, dt);
    if (L.total > kNoAllocScratchBytes) return MOE_ERR_UNSUPPORTED;
    char* base = nullptr;
    if (scratch_address(stream, &base) != hipSuccess) return MOE_ERR_HIP;
    FwdBuffers b;
    b.ids = (int32_t*)(base + L.ids);
    b.w = (float*)(base + L.w);
    b.off = (int32_t*)(base + L.offsets);
    b.inv = (int32_t*)(base + L.inv);
    b.row_token = (int32_t*)(base + L.row_token);
    b.partial = (int32_t*)(base + L.partial);
    b.x_perm = L.gather ? nullptr : base + L.x_perm;
    b.y_perm = (float*)(base + L.y_perm);
    b.y_sh = fs > 0 ? (float*)(base + L.y_sh) : nullptr;
    b.ffn = base + L.ffn;
    b.route = base + L.route;
    return enqueue_forward(x, Wr, bias, W1, W2, W1s, W2s, fs, T, H, F, E, k, drop_thresh, dt, y, out_dt, topk_ids,
                           topk_w, expert_offsets, inv, b, stream);
}

size_t moe_fp8_weight_bytes(int E, int K, int N) {
    if (E < 1 || K < 1 || N < 1 || E > kMaxExperts || K % 64 != 0) return 0;
    return (size_t)moe::fp8_weight_bytes(E, K, N);
}

int moe_quantize_fp8(const void* W, int E, int K, int N, moe_dtype_t dt, uint8_t* Wq, float* scales,
                     hipStream_t stream) {
    if (!valid_dtype(dt)) return MOE_ERR_INVALID_ARG;
    if (E < 1 || K < 1 || N < 1) return MOE_ERR_INVALID_ARG;
    if (E > kMaxExperts || K % 64 != 0) return MOE_ERR_UNSUPPORTED;
    if ((long long)E * ((N + 127) / 128) * (K / 64) >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;  // tile grid
    if (!W || !Wq || !scales) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_quantize_fp8(W, E, K, N, (Dtype)dt, Wq, scales, stream));
}

int moe_grouped_ffn_fp8(const void* x_perm, const int32_t* expert_offsets, const uint8_t* W1q, const float* W1_scale,
                        const uint8_t* W2q, const float* W2_scale, int T, int H, int F, int E, int k, float* y_perm,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
    if (F < 1) return MOE_ERR_INVALID_ARG;
    int st = check_sizes(T, H, F, E, k);
    if (st != MOE_OK) return st;
    if (!moe::ffn_fp8_ok(H, F)) return MOE_ERR_UNSUPPORTED;
    if (!x_perm || !expert_offsets || !W1q || !W1_scale || !W2q || !W2_scale || !y_perm || !ws)
        return MOE_ERR_INVALID_ARG;
    const FfnLayout L = ffn_layout(T, F, k, 0, MOE_BF16);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    const int rows = T * k;
    const moe::TileCfg cfg = moe::choose_tile(rows, E);
    void* h = (char*)ws + L.h;
    MOE_TRY(moe::launch_ffn_up_fp8(x_perm, nullptr, expert_offsets, E, rows, W1q, W1_scale, H, F, cfg, h, stream));
    return hip_status(
        moe::launch_ffn_down_fp8(h, expert_offsets, E, rows, W2q, W2_scale, F, H, cfg, false, y_perm, 0, stream));
}

int moe_forward_fp8(const void* x, const void* Wr, const float* bias, const uint8_t* W1q, const float* W1_scale,
                    const uint8_t* W2q, const float* W2_scale, int T, int H, int F, int E, int k, float drop_thresh,
                    void* y, moe_dtype_t out_dt, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                    int32_t* inv, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!valid_dtype(out_dt)) return MOE_ERR_INVALID_ARG;
    if (F < 1) return MOE_ERR_INVALID_ARG;
    int st = check_sizes(T, H, F, E, k);
    if (st != MOE_OK) return st;
    if ((st = check_drop(drop_thresh, k)) != MOE_OK) return st;
    if (!moe::ffn_fp8_ok(H, F)) return MOE_ERR_UNSUPPORTED;
    if (!x || !Wr || !W1q || !W1_scale || !W2q || !W2_scale || !y || !ws) return MOE_ERR_INVALID_ARG;
    const FwdLayout L = fwd_layout(T, H, F, E, k, 0, MOE_BF16);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    char* base = (char*)ws;
    int32_t* ids = topk_ids ? topk_ids : (int32_t*)(base + L.ids);
    float* w = topk_w ? topk_w : (float*)(base + L.w);
    int32_t* off = expert_offsets ? expert_offsets : (int32_t*)(base + L.offsets);
    int32_t* iv = inv ? inv : (int32_t*)(base + L.inv);
    int32_t* row_token = (int32_t*)(base + L.row_token);
    int32_t* partial = (int32_t*)(base + L.partial);
    void* y_planes = base + L.y_perm;
    void* h = base + L.ffn + ffn_layout(T, F, k, 0, MOE_BF16).h;
    const int rows = T * k;
    const moe::TileCfg cfg = moe::choose_tile(rows, E);
    // the W1 launch gathers x rows through row_token (no permuted copy); the W2 launch writes block-scaled fp16 y_perm
    if ((st = enqueue_route_permute(x, Wr, bias, T, H, E, k, drop_thresh, MOE_BF16, ids, w, base + L.route, nullptr,
                                    off, row_token, iv, partial, false, stream)) != MOE_OK)
        return st;
    MOE_TRY(moe::launch_ffn_up_fp8(x, row_token, off, E, rows, W1q, W1_scale, H, F, cfg, h, stream));
    MOE_TRY(moe::launch_ffn_down_fp8(h, off, E, rows, W2q, W2_scale, F, H, cfg, true, y_planes, rows, stream));
    return hip_status(moe::launch_combine_packed(y_planes, rows, iv, w, nullptr, T, H, k, (moe::Dtype)out_dt, y,
                                                 stream));
}

size_t moe_mxfp8_weight_bytes(int E, int K, int N) {
    if (E < 1 || K < 1 || N < 1 || E > kMaxExperts || K % 128 != 0) return 0;
    return (size_t)moe::mx_weight_bytes(E, K, N);
}

size_t moe_mxfp8_scale_bytes(int E, int K, int N) {
    if (E < 1 || K < 1 || N < 1 || E > kMaxExperts || K % 128 != 0) return 0;
    return (size_t)moe::mx_weight_scale_bytes(E, K, N);
}

int moe_quantize_mxfp8(const void* W, int E, int K, int N, moe_dtype_t dt, uint8_t* Wq, uint8_t* W_scale,
                       hipStream_t stream) {
    if (!valid_dtype(dt)) return MOE_ERR_INVALID_ARG;
    if (E < 1 || K < 1 || N < 1) return MOE_ERR_INVALID_ARG;
    if (E > kMaxExperts || K % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if ((long long)E * ((N + 127) / 128) * (K / 128) >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
    if (!W || !Wq || !W_scale) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_quantize_mx_weights(W, E, K, N, (Dtype)dt, Wq, W_scale, stream));
}

int moe_quantize_mxfp8_rows(const void* x, int T, int H, moe_dtype_t dt, uint8_t* xq, uint8_t* x_scale,
                            hipStream_t stream) {
    if (!valid_dtype(dt)) return MOE_ERR_INVALID_ARG;
    if (T < 1 || H < 1) return MOE_ERR_INVALID_ARG;
    if (H % 128 != 0 || (long long)T * H >= (1LL << 40)) return MOE_ERR_UNSUPPORTED;
    if (!x || !xq || !x_scale) return MOE_ERR_INVALID_ARG;
    return hip_status(
        moe::launch_quantize_mx_rows(x, T, H, (Dtype)dt, xq, x_scale, stream));
}

size_t moe_grouped_ffn_mxfp8_workspace_bytes(int T, int H, int k) {
    if (T < 1 || H < 1 || k < 1 || k > kMaxK || H % 128 != 0) return 0;
    return align_up((size_t)T * H) + align_up((size_t)(H / 128) * T * 4);
}

int moe_grouped_ffn_mxfp8(const void* x, const int32_t* row_token, const int32_t* expert_offsets,
                          const uint8_t* W1q, const uint8_t* W1_scale, const uint8_t* W2q, const uint8_t* W2_scale,
                          int T, int H, int F, int E, int k, uint8_t* h_codes, uint8_t* h_scale, float* y_perm,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
    if (F < 1) return MOE_ERR_INVALID_ARG;
    int st = check_sizes(T, H, F, E, k);
    if (st != MOE_OK) return st;
    if (!moe::ffn_mx_ok(H, F)) return MOE_ERR_UNSUPPORTED;
    if ((long long)T * k * F >= (1LL << 31) || (long long)T * k * H * 4 >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
    if (!x || !row_token || !expert_offsets || !W1q || !W1_scale || !W2q || !W2_scale || !h_codes || !h_scale ||
        !y_perm || !ws)
        return MOE_ERR_INVALID_ARG;
    if (ws_bytes < moe_grouped_ffn_mxfp8_workspace_bytes(T, H, k)) return MOE_ERR_WORKSPACE;
    const long rows = (long)T * k;
    uint8_t* xq = (uint8_t*)ws;
    uint8_t* xs = xq + align_up((size_t)T * H);
    // quantise the token rows once; the W1 launch gathers their codes through row_token
    MOE_TRY(moe::launch_quantize_mx_rows(x, T, H, moe::kBF16, xq, xs, stream));
    MOE_TRY(moe::launch_ffn_up_mx(xq, xs, T, row_token, expert_offsets, E, (int)rows, W1q, W1_scale, H, F, h_codes,
                                  h_scale, rows, stream));
    return hip_status(moe::launch_ffn_down_mx(h_codes, h_scale, rows, expert_offsets, E, (int)rows, W2q, W2_scale, F,
                                              H, false, y_perm, stream));
}

size_t moe_mxfp8_workspace_bytes(int T, int H, int F, int E, int k) {
    if (check_sizes(T, H, F, E, k) != MOE_OK || F < 1 || !moe::ffn_mx_ok(H, F)) return 0;
    return mx_layout(T, H, F, E, k).total;
}

int moe_forward_mxfp8(const void* x, const void* Wr, const float* bias, const uint8_t* W1q, const uint8_t* W1_scale,
                      const uint8_t* W2q, const uint8_t* W2_scale, int T, int H, int F, int E, int k,
                      float drop_thresh, void* y, moe_dtype_t out_dt, int32_t* topk_ids, float* topk_w,
                      int32_t* expert_offsets, int32_t* inv, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!valid_dtype(out_dt)) return MOE_ERR_INVALID_ARG;
    if (F < 1) return MOE_ERR_INVALID_ARG;
    int st = check_sizes(T, H, F, E, k);
    if (st != MOE_OK) return st;
    if ((st = check_drop(drop_thresh, k)) != MOE_OK) return st;
    if (!moe::ffn_mx_ok(H, F)) return MOE_ERR_UNSUPPORTED;
    if ((long long)T * k * F >= (1LL << 31) || (long long)T * k * H * 2 >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
    if (!x || !Wr || !W1q || !W1_scale || !W2q || !W2_scale || !y || !ws) return MOE_ERR_INVALID_ARG;
    const MxLayout L = mx_layout(T, H, F, E, k);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    char* base = (char*)ws;
    int32_t* ids = topk_ids ? topk_ids : (int32_t*)(base + L.ids);
    float* w = topk_w ? topk_w : (float*)(base + L.w);
    int32_t* off = expert_offsets ? expert_offsets : (int32_t*)(base + L.offsets);
    int32_t* iv = inv ? inv : (int32_t*)(base + L.inv);
    int32_t* row_token = (int32_t*)(base + L.row_token);
    const long rows = (long)T * k;
    uint8_t* xq = (uint8_t*)(base + L.xq);
    uint8_t* xs = (uint8_t*)(base + L.xs);
    // the router keeps bf16 x; the experts read x quantised to MX once per token (gathered by the W1 launch)
    if ((st = enqueue_route_permute(x, Wr, bias, T, H, E, k, drop_thresh, MOE_BF16, ids, w, base + L.route, nullptr,
                                    off, row_token, iv, (int32_t*)(base + L.partial), false, stream)) != MOE_OK)
        return st;
    MOE_TRY(moe::launch_quantize_mx_rows(x, T, H, moe::kBF16, xq, xs, stream));
    MOE_TRY(moe::launch_ffn_up_mx(xq, xs, T, row_token, off, E, (int)rows, W1q, W1_scale, H, F, base + L.hq,
                                  base + L.hs, rows, stream));
    MOE_TRY(moe::launch_ffn_down_mx(base + L.hq, base + L.hs, rows, off, E, (int)rows, W2q, W2_scale, F, H, true,
                                    base + L.y, stream));
    return hip_status(
        moe::launch_combine_packed(base + L.y, rows, iv, w, nullptr, T, H, k, (moe::Dtype)out_dt, y, stream));
}

int moe_calibrate_mfma_bf16(int workgroups, int waves_per_workgroup, int iters, int operands, float* sink,
                            hipStream_t stream) {
    if (workgroups < 1 || waves_per_workgroup < 1 || waves_per_workgroup > 8 || iters < 1) return MOE_ERR_INVALID_ARG;
    if (!sink || operands < 0 || operands > 1) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_calibrate_mfma(workgroups, waves_per_workgroup, iters, operands, sink, stream));
}

int moe_calibrate_stream_read(const void* buf, size_t bytes, int workgroups, float* sink, hipStream_t stream) {
    if (workgroups < 1 || bytes < 16 || bytes % 16 != 0) return MOE_ERR_INVALID_ARG;
    if (!buf || !sink) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_calibrate_read(buf, (long)bytes, workgroups, sink, stream));
}

int moe_calibrate_gemm_kstep(const void* src, size_t span, int workgroups, int steps, int mode, float* sink,
                             hipStream_t stream) {
    if (workgroups < 1 || steps < 1 || mode < 0 || mode > 2) return MOE_ERR_INVALID_ARG;
    if (mode >= 1 && (!src || span < 32768 || span % 16 != 0)) return MOE_ERR_INVALID_ARG;
    if (!sink) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_calibrate_kstep(src, (long)span, workgroups, steps, mode, sink, stream));
}

}  // extern "C"
