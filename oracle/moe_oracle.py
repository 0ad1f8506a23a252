"""Plain fp64 CPU oracle of one MoE feed-forward layer's forward pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. It shares no code,
tables or helpers with the HIP library.

Sources (pages are cited by title/address and section):

[P1] "MoE大模型的智能调度：从1.8万亿参数到每token仅激活2%的工程真相"
     (www.jsqmd.com/news/1091713), section 2.2, the three layers: the routing
     layer (scores per expert; keep the top-k logits and softmax them; zero a
     weight under the 0.05 threshold and renormalise), the expert layer (every
     expert is an independent two-layer FFN) and the fusion layer (the output
     is the gate-weighted sum of the chosen experts' outputs).
     Section 4.1 (model loading and memory budget): the resident experts'
     weights are quantised to 8 bits.
     Section 3.2, second routing pitfall: a per-expert selection capacity of
     tokens*k/experts*1.2; over-capacity experts get -inf and the token
     chooses again (the capacity-limited routing variant).
[P3] "跟随一个Token走完路由、分发、专家计算到合并和多机放置的整条路径"
     (m.lsln.cn/news/228042):
     - section "MoE层的结构与token路由" (MoE layer structure and token
       routing): the layer output is the sum, over the selected experts only,
       of the routing weight times that expert's output; shared experts take
       every token and are not scored by the router;
     - section "一个批次如何变成各专家专属的矩阵" (how a batch becomes
       per-expert matrices): an assignment is (token vector, expert, weight);
       assignments are grouped per expert into matrices, the source token id is
       kept beside each row, each token's results are scaled by their weights
       and added; an expert batch counts assignments, so top-k gives k rows
       per token;
     - section "单机MoE执行流水线" (single-GPU MoE pipeline): score, top-k,
       permute rows into contiguous per-expert blocks while recording an
       inverse map, run the grouped GEMM, the activation and the output
       projection, then restore token order with the inverse map, apply the
       routing weights and accumulate the contributions of each token.

Readings where the pages leave a step open (each is listed with its reason in
the design notes of the repository):

* router: linear, ``logits = x @ Wr + b``; no temperature;
* top-k order: logit descending, ties to the lower expert id;
* weights: softmax over the k selected logits (equal, in exact arithmetic, to
  a softmax over all experts restricted to the selection and renormalised);
* drop threshold tau: a renormalised weight strictly below tau is set to zero
  and the survivors are renormalised once; a dropped assignment is not
  dispatched;
* slot order inside a token: ascending expert id (the worked example lists
  each token's experts by id, not by weight);
* row order inside an expert: ascending token id (a stable counting sort);
* expert FFN: ``silu(x @ W1[e]) @ W2[e]``, silu(u) = u / (1 + exp(-u)), no
  biases; shared expert: the same form with weight 1;
* low-precision experts: fp8 e4m3 codes with one fp32 scale per expert and
  output column (max|W|/448), round-to-nearest-even in float32; the layer is
  evaluated with the dequantised weights;
* MX fp8 (activations and weights in 8 bits on the fp8 matrix cores): OCP MX
  E4M3 blocks of 32 along each product's reduction axis, shared scale
  2^(floor(log2 amax) - 8); the token rows are quantised before dispatch, the
  expert's SiLU output is re-quantised before the second product;
* capacity-limited routing: capacity = ceil(T*k/E*factor); tokens choose in
  ascending id among experts not yet full (serial priority by token id);
  capacity counts selections, before any drop.

Every function here is pinned by the CPU tests (worked example, drop case,
library special cases, dense brute force, invariants); none is unpinned.
"""
from __future__ import annotations

import dataclasses
import math
import time
from typing import Callable, Optional, Sequence, Union


import numpy as np

ArrayOrGetter = Union[np.ndarray, Callable[[int], np.ndarray]]


@dataclasses.dataclass
class RouteResult:
    ids: np.ndarray      # [T,k] int64, ascending expert id per token
    w: np.ndarray        # [T,k] float64, 0.0 where dropped
    keep: np.ndarray     # [T,k] bool
    logits: np.ndarray   # [T,E] float64
    gap: np.ndarray      # [T] k-th minus (k+1)-th largest logit (inf when k == E)


@dataclasses.dataclass
class DispatchResult:
    counts: np.ndarray     # [E] int64
    offsets: np.ndarray    # [E+1] int64
    row_token: np.ndarray  # [A] int64
    inv: np.ndarray        # [T,k] int64, -1 for a dropped slot


@dataclasses.dataclass
class ForwardResult:
    route: RouteResult
    dispatch: DispatchResult
    x_perm: np.ndarray
    y_perm: np.ndarray
    y_shared: Optional[np.ndarray]
    y: np.ndarray
    times: dict


def _w(getter: ArrayOrGetter, e: int) -> np.ndarray:
    return getter(e) if callable(getter) else getter[e]


def router_logits(x: np.ndarray, Wr: np.ndarray, b: Optional[np.ndarray] = None) -> np.ndarray:
    """Router scores, one per (token, expert): ``x @ Wr + b`` in fp64.

    [P1] section 2.2, routing layer step 1; [P3] "单机MoE执行流水线" (the
    router first produces a score for every candidate expert).
    """
    s = np.asarray(x, dtype=np.float64) @ np.asarray(Wr, dtype=np.float64)
    if b is not None:
        s = s + np.asarray(b, dtype=np.float64)[None, :]
    return s


def select_topk(logits: np.ndarray, k: int):
    """The k experts with the largest logits, ties to the lower id.

    Returns (ids sorted ascending [T,k], gap [T]). [P1] section 2.2, routing
    layer step 2 (take the top-k logits); [P3] "单机MoE执行流水线" (top-k
    keeps the selected expert indices).
    """
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.broadcast_to(np.arange(E), (T, E))
    # lexsort: last key is primary -> logit descending, then id ascending
    order = np.lexsort((ids, -logits), axis=1)
    chosen = order[:, :k]
    ranked = np.take_along_axis(logits, order, axis=1)
    gap = ranked[:, k - 1] - ranked[:, k] if k < E else np.full(T, np.inf)
    return np.sort(chosen, axis=1), gap


def route(x, Wr, b, k: int, drop_thresh: float = 0.0) -> RouteResult:
    """Top-k routing with softmax weights over the selection and an optional drop.

    [P1] section 2.2, routing layer steps 1-3: score, softmax the top-k
    logits into weights, zero a weight under the threshold and renormalise.
    Slots are returned in ascending expert id.
    """
    logits = router_logits(x, Wr, b)
    ids, gap = select_topk(logits, k)
    w, keep = selection_weights(logits, ids, drop_thresh)
    return RouteResult(ids=ids.astype(np.int64), w=w, keep=keep, logits=logits, gap=gap)


def selection_weights(logits: np.ndarray, ids: np.ndarray, drop_thresh: float = 0.0):
    """Softmax over each token's selected logits, then the optional drop.

    [P1] section 2.2, routing layer steps 2-3: the selected logits become
    weights through a softmax; a weight below the threshold is zeroed and the
    others renormalised (strictly below is dropped; one pass is a fixed point
    because the survivors only grow).
    """
    sel = np.take_along_axis(np.asarray(logits, dtype=np.float64), ids, axis=1)
    m = sel.max(axis=1, keepdims=True)
    p = np.exp(sel - m)
    w = p / p.sum(axis=1, keepdims=True)
    keep = np.ones_like(w, dtype=bool)
    if drop_thresh > 0.0:
        keep = w >= drop_thresh
        w = np.where(keep, w, 0.0)
        w = w / w.sum(axis=1, keepdims=True)
    return w, keep


# ------------------------------------------------- low-precision expert weights --
# [P1] section 4.1 (model loading and memory budget): the resident experts'
# FFN weights are quantised to 8 bits (INT8 there) because their
# distribution is concentrated, halving their memory. Reading taken here for
# MI355X: 8-bit OCP fp8 e4m3 codes with one fp32 scale per expert and output
# column, s = max_k |W[e,k,n]| / 448 (448 = largest finite e4m3 value; an
# all-zero column gets s = 1), codes = e4m3 round-to-nearest-even of W / s,
# both steps in float32. The quantised layer is the layer evaluated with the
# dequantised weights s * value(code).

def e4m3_values() -> np.ndarray:
    """Value of every OCP fp8 e4m3 code (sign, 4 exponent bits with bias 7,
    3 mantissa bits; exponent 0 is subnormal; 0x7F/0xFF are NaN; no inf)."""
    v = np.empty(256, dtype=np.float64)
    for c in range(256):
        sgn, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v[c] = np.nan
            continue
        mag = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        v[c] = -mag if sgn else mag
    return v


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest finite e4m3 value to each x, ties to the even code, saturating at
    448; the sign bit is the sign of x (so -0.0 -> 0x80). x must be finite.
    The two candidates are the neighbouring codes of |x| in the increasing
    table of the 127 non-negative finite values."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode: non-finite input")
    mags = e4m3_values()[:0x7F]                        # codes 0x00..0x7E, increasing
    a = np.minimum(np.abs(x), mags[-1])                # beyond 448 the nearest finite value is 448
    hi = np.minimum(np.searchsorted(mags, a, side="left"), 0x7E)   # first code with value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    sign = np.signbit(x).astype(np.int64) << 7
    return (pick | sign).astype(np.uint8)


def quantize_fp8(W: np.ndarray):
    """Per expert and output column: s = max|W| / 448 and codes = e4m3(W / s), in
    float32. W: [E,K,N] (any float dtype, converted exactly to float32).
    Returns (codes uint8 [E,K,N], scales float32 [E,N])."""
    W32 = np.asarray(W, dtype=np.float32)
    amax = np.abs(W32).max(axis=1)                       # [E,N], exact
    s = (amax / np.float32(448.0)).astype(np.float32)    # one IEEE float32 division
    s = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    ratio = (W32 / s[:, None, :]).astype(np.float32)     # float32 division, rounded once
    return e4m3_encode(ratio), s


def dequantize_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W_deq[e,k,n] = scales[e,n] * value(codes[e,k,n]) in float64."""
    return e4m3_values()[codes.astype(np.int64)] * scales.astype(np.float64)[:, None, :]


# MX (microscaling) fp8: activations as well as weights in 8 bits, so that the
# products run on the fp8 matrix cores. Reading: the OCP MX block format with
# E4M3 elements -- every 32 consecutive values along the reduction axis share
# one power-of-two scale X = 2^(floor(log2(amax)) - 8) (8 = exponent of the
# largest E4M3 power of two, 2^8 <= 448 < 2^9), stored as a biased exponent
# byte (E8M0, bias 127); each value is encoded as e4m3(V / X) with the same
# rounding and saturation as above (values in [448, 512)·X clamp to 448·X).
# An all-zero block has X = 1. V / X is exact in float32 (a power-of-two
# scaling of a float32 value), so the codes depend on the float32 inputs only.

MX_BLOCK = 32
MX_EMAX_E4M3 = 8


def mx_scale_exponents(amax: np.ndarray) -> np.ndarray:
    """Unbiased shared exponent floor(log2(amax)) - 8 per block (0 for amax == 0),
    clamped to the E8M0 range [-127, 127]."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)            # amax = m * 2^e, 0.5 <= m < 1: floor(log2(amax)) = e - 1
    x = np.where(amax > 0, e - 1 - MX_EMAX_E4M3, 0)
    return np.clip(x, -127, 127).astype(np.int64)


def quantize_mx(V: np.ndarray, axis: int):
    """MX E4M3 of V (any float dtype, converted exactly to float32) with blocks of
    32 consecutive elements along ``axis`` (its length a multiple of 32).
    Returns (codes uint8, same shape as V; scale bytes uint8 with that axis
    divided by 32, value = unbiased exponent + 127)."""
    V32 = np.asarray(V, dtype=np.float32)
    Vm = np.moveaxis(V32, axis, -1)
    n = Vm.shape[-1]
    if n % MX_BLOCK != 0:
        raise ValueError("quantize_mx: axis length must be a multiple of 32")
    blocks = Vm.reshape(Vm.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    xexp = mx_scale_exponents(np.abs(blocks).max(axis=-1))
    scaled = blocks.astype(np.float64) * np.ldexp(1.0, -xexp)[..., None]   # exact
    codes = e4m3_encode(scaled).reshape(Vm.shape)
    return np.moveaxis(codes, -1, axis), np.moveaxis((xexp + 127).astype(np.uint8), -1, axis)


def dequantize_mx(codes: np.ndarray, scale_bytes: np.ndarray, axis: int) -> np.ndarray:
    """value(code) * 2^(scale byte - 127), blocks of 32 along ``axis``, float64."""
    vals = e4m3_values()[np.asarray(codes).astype(np.int64)]
    x = np.repeat(np.ldexp(1.0, scale_bytes.astype(np.int64) - 127), MX_BLOCK, axis=axis)
    return vals * x


def expert_ffn_mx(rows: np.ndarray, W1e: np.ndarray, W2e: np.ndarray) -> np.ndarray:
    """One expert on MX-quantised operands: rows (already dequantised MX
    activations) @ W1e (dequantised), SiLU, the result re-quantised to MX along
    its F axis (the W2 product's reduction axis) and dequantised, @ W2e."""
    h = silu(rows @ W1e)
    hq, hs = quantize_mx(h, axis=1)
    return dequantize_mx(hq, hs, axis=1) @ W2e


# ------------------------------------------------- capacity-limited routing --
# [P1] section 3.2, second pitfall ("Top-k 选择忽略专家容量"): every expert gets a
# selection limit capacity = tokens * k / experts * 1.2; an expert chosen more
# often than that has its logit set to -inf for the excess tokens, which then
# choose again. Reading taken here: tokens have priority by ascending id, so
# token t picks its k best experts among those that the tokens before it have
# not yet filled (a fixed, deterministic order; ties to the lower id as in
# plain routing). Capacity counts selections, before any drop.

def capacity_slots(T: int, k: int, E: int, factor: float) -> int:
    """ceil(T*k/E*factor), evaluated in float64 in that order."""
    return int(math.ceil(T * k / E * float(factor)))


def capacity_feasible(T: int, k: int, E: int, cap: int) -> bool:
    """A sufficient condition for every token to find k experts with room,
    checkable before routing: at most floor(T*k/cap) experts can ever be full,
    so at least E minus that many always have room."""
    return cap >= 1 and E - (T * k) // cap >= k


def select_capacity(logits: np.ndarray, k: int, cap: int) -> np.ndarray:
    """Capacity-limited top-k: ids [T,k] ascending per row.

    Tokens in ascending id; each takes the k largest logits among experts
    whose selection count is still below cap (full experts are treated as
    -inf); ties go to the lower expert id. The comparisons are made on the
    logits exactly as given (pass float32 values to decide in float32).
    """
    T, E = logits.shape
    count = np.zeros(E, dtype=np.int64)
    ids = np.zeros((T, k), dtype=np.int64)
    eid = np.arange(E)
    for t in range(T):
        room = count < cap
        if room.sum() < k:
            raise ValueError(f"token {t}: fewer than k experts have room")
        cand = eid[room]
        vals = logits[t, room]
        order = np.lexsort((cand, -vals.astype(np.float64)))  # logit descending, then id ascending
        chosen = np.sort(cand[order[:k]])
        ids[t] = chosen
        count[chosen] += 1
    return ids


def route_capacity(x, Wr, b, k: int, drop_thresh: float, factor: float) -> RouteResult:
    """Capacity-limited routing: fp64 logits, select_capacity, softmax over the
    selected logits, optional drop. gap = per token, its k-th minus (k+1)-th
    largest logit among the experts that had room when it chose."""
    logits = router_logits(x, Wr, b)
    T, E = logits.shape
    cap = capacity_slots(T, k, E, factor)
    ids = select_capacity(logits, k, cap)
    w, keep = selection_weights(logits, ids, drop_thresh)
    return RouteResult(ids=ids, w=w, keep=keep, logits=logits, gap=capacity_gaps(logits, ids, cap))


def capacity_gaps(logits: np.ndarray, ids: np.ndarray, cap: int) -> np.ndarray:
    """For each token: smallest selected logit minus largest unselected logit
    among the experts that still had room when the token chose (inf if none)."""
    T, E = logits.shape
    count = np.zeros(E, dtype=np.int64)
    gap = np.full(T, np.inf)
    for t in range(T):
        room = count < cap
        sel = np.zeros(E, dtype=bool)
        sel[ids[t]] = True
        other = room & ~sel
        if other.any():
            gap[t] = logits[t, ids[t]].min() - logits[t, other].max()
        count[ids[t]] += 1
    return gap


def dispatch(ids: np.ndarray, keep: np.ndarray, E: int) -> DispatchResult:
    """Group the kept assignments by expert (a stable counting sort).

    [P3] "一个批次如何变成各专家专属的矩阵": assignments are grouped per
    expert, each group is one matrix, and the source token id is kept beside
    each row; [P3] "单机MoE执行流水线": the permute writes rows in expert order
    and records an inverse map for the combine. Rows of expert e are its kept
    assignments in ascending token id; inv[t, j] is the row of slot j of
    token t, or -1 when that slot was dropped.
    """
    T, k = ids.shape
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if keep[t, j]:
                counts[ids[t, j]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    nxt = offsets[:-1].copy()
    A = int(offsets[-1])
    row_token = np.full(A, -1, dtype=np.int64)
    inv = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if keep[t, j]:
                e = ids[t, j]
                r = nxt[e]
                nxt[e] += 1
                row_token[r] = t
                inv[t, j] = r
    return DispatchResult(counts=counts, offsets=offsets, row_token=row_token, inv=inv)


def silu(u: np.ndarray) -> np.ndarray:
    """u * sigmoid(u) = u / (1 + exp(-u))."""
    with np.errstate(over="ignore"):
        return u / (1.0 + np.exp(-u))


def expert_ffn(rows: np.ndarray, W1e: np.ndarray, W2e: np.ndarray) -> np.ndarray:
    """One expert: a two-layer FFN, ``silu(rows @ W1e) @ W2e`` in fp64.

    [P1] section 2.2, expert layer (independent two-layer FFNs with their own
    W1, W2); [P3] "单机MoE执行流水线" (each expert applies its activation and
    output projection).
    """
    rows = np.asarray(rows, dtype=np.float64)
    h = silu(rows @ np.asarray(W1e, dtype=np.float64))
    return h @ np.asarray(W2e, dtype=np.float64)


def grouped_ffn(x_perm: np.ndarray, offsets: np.ndarray, W1: ArrayOrGetter, W2: ArrayOrGetter) -> np.ndarray:
    """Apply expert e's FFN to its contiguous block of rows [offsets[e], offsets[e+1]).

    [P3] "单机MoE执行流水线": the grouped GEMM runs all expert matrices,
    whose row counts differ, without changing their contents.
    """
    E = len(offsets) - 1
    H_out = None
    out = None
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        ye = expert_ffn(x_perm[a:b], _w(W1, e), _w(W2, e))
        if out is None:
            H_out = ye.shape[1]
            out = np.zeros((x_perm.shape[0], H_out), dtype=np.float64)
        out[a:b] = ye
    if out is None:
        out = np.zeros((x_perm.shape[0], x_perm.shape[1]), dtype=np.float64)
    return out


def shared_ffn(x: np.ndarray, W1s: np.ndarray, W2s: np.ndarray) -> np.ndarray:
    """The always-on shared expert: same FFN form, applied to every token.

    [P3] "MoE层的结构与token路由": shared experts ignore the router's scores
    and every token passes through them.
    """
    return expert_ffn(x, W1s, W2s)


def combine(y_perm: np.ndarray, inv: np.ndarray, w: np.ndarray, y_shared: Optional[np.ndarray] = None,
            T: Optional[int] = None) -> np.ndarray:
    """Restore token order, scale by the routing weights and add per token.

    [P1] section 2.2, fusion layer (gated sum of expert outputs); [P3]
    "一个批次如何变成各专家专属的矩阵" (each of a token's results is scaled by
    its weight and the scaled results are added); [P3] "单机MoE执行流水线"
    (the inverse map restores token order). The shared expert's output, when
    present, is added with weight 1.
    """
    T = inv.shape[0] if T is None else T
    H = y_perm.shape[1]
    y = np.zeros((T, H), dtype=np.float64)
    for j in range(inv.shape[1]):
        r = inv[:, j]
        m = r >= 0
        y[m] += w[m, j][:, None] * y_perm[r[m]]
    if y_shared is not None:
        y += y_shared
    return y


def forward(x, Wr, b, W1: ArrayOrGetter, W2: ArrayOrGetter, k: int, drop_thresh: float = 0.0,
            W1s=None, W2s=None) -> ForwardResult:
    """The whole layer in the pipeline order of [P3] "单机MoE执行流水线", with stage timers."""
    times = {}
    x = np.asarray(x, dtype=np.float64)
    E = (Wr.shape[1])
    t0 = time.perf_counter()
    r = route(x, Wr, b, k, drop_thresh)
    t1 = time.perf_counter()
    d = dispatch(r.ids, r.keep, E)
    x_perm = x[d.row_token]
    t2 = time.perf_counter()
    y_perm = grouped_ffn(x_perm, d.offsets, W1, W2)
    y_sh = shared_ffn(x, W1s, W2s) if W1s is not None else None
    t3 = time.perf_counter()
    y = combine(y_perm, d.inv, r.w, y_sh)
    t4 = time.perf_counter()
    times.update(route=t1 - t0, permute=t2 - t1, ffn=t3 - t2, combine=t4 - t3)
    return ForwardResult(route=r, dispatch=d, x_perm=x_perm, y_perm=y_perm, y_shared=y_sh, y=y, times=times)


def forward_tokens(tokens: Sequence[int], x, Wr, b, W1: ArrayOrGetter, W2: ArrayOrGetter, k: int,
                   drop_thresh: float = 0.0, W1s=None, W2s=None, mx: bool = False):
    """Layer output for selected tokens only, by the layer equation.

    [P3] "MoE层的结构与token路由": y(x) is the sum over the selected experts
    of w_e(x) * E_e(x). Returns (ids, w, keep, y) for ``tokens``. Each
    expert's weights are fetched once and applied to the sampled tokens that
    chose it; the per-token sum then runs in slot order.

    mx=True: the MX fp8 layer -- routing on x as given, the experts on the
    token rows quantised to MX along H (before dispatch) and dequantised, with
    expert_ffn_mx (W1, W2 are then the dequantised MX weights).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    xs = np.asarray(x, dtype=np.float64)[tokens]
    r = route(xs, Wr, b, k, drop_thresh)
    n = len(tokens)
    H = xs.shape[1]
    xe = dequantize_mx(*quantize_mx(xs, axis=1), axis=1) if mx else xs
    ffn = expert_ffn_mx if mx else expert_ffn
    contrib = np.zeros((n, k, H), dtype=np.float64)
    for e in np.unique(r.ids[r.keep]):
        which = np.argwhere((r.ids == e) & r.keep)
        ye = ffn(xe[which[:, 0]], _w(W1, int(e)), _w(W2, int(e)))
        contrib[which[:, 0], which[:, 1]] = ye
    y = np.zeros((n, H), dtype=np.float64)
    for j in range(k):
        y += r.w[:, j][:, None] * contrib[:, j]
    if W1s is not None:
        y += shared_ffn(xs, W1s, W2s)
    return r.ids, r.w, r.keep, y


def dense_bruteforce(x, Wr, b, W1, W2, k: int, drop_thresh: float = 0.0, W1s=None, W2s=None) -> np.ndarray:
    """Every expert on every token, masked by the routing weights (zero off S(x)).

    [P3] "MoE层的结构与token路由": the sum covers only the selected experts,
    so a dense sum over all experts with a weight that is zero outside S(x)
    gives the same y without any dispatch or inverse map.
    """
    x = np.asarray(x, dtype=np.float64)
    E = Wr.shape[1]
    r = route(x, Wr, b, k, drop_thresh)
    T = x.shape[0]
    mask = np.zeros((T, E), dtype=np.float64)
    for j in range(k):
        mask[np.arange(T), r.ids[:, j]] = r.w[:, j]
    y = np.zeros((T, _w(W2, 0).shape[1]), dtype=np.float64)
    for e in range(E):
        y += mask[:, e:e + 1] * expert_ffn(x, _w(W1, e), _w(W2, e))
    if W1s is not None:
        y += shared_ffn(x, W1s, W2s)
    return y
