"""Seeded synthetic inputs for the single-GPU MoE-layer forward.

This package only draws and rounds input arrays; it never produces an
expected value. Both the fp64 CPU oracle (``oracle/``) and the GPU library
read what it writes, so every parity check sees the same bits on both sides.

Recipe (shapes follow the workloads named in ``CONFIGS``):

* ``x ~ N(0, 1)``; router ``Wr[H,E] ~ N(0, 1/sqrt(H))``;
  ``W1[E,H,F] ~ N(0, 1/sqrt(H))``; ``W2[E,F,H] ~ N(0, 1/sqrt(F))``; the shared
  expert uses the same rule with its own hidden width ``Fs``. The second
  parameter is the standard deviation.
* Deviates come from ``philox_normal.c`` (Philox4x32-10 + Box-Muller), keyed
  on (seed, tensor id) with the element index and a re-draw attempt in the
  counter, so any single token row can be re-drawn without touching the rest.
* Values are rounded once to the storage type: fp32, or fp32 then bf16, both
  round-to-nearest-even. bf16 arrays are held as raw ``uint16`` bit patterns.
* Skewed-load workload: a router bias ``b_e = beta * ln p_{pi(e)}`` with
  ``p_r`` proportional to ``r^-1.2`` (Zipf) and ``pi`` a seeded permutation of
  the experts; ``beta`` is fitted by bisection so that the hottest expert
  takes 35-40% of the top-k assignments, the imbalance page 2 reports in its
  load-balance discussion (section 2.3) for an 8-expert model.
* Near-tie conditioning: a token row is re-drawn while the gap between its
  k-th and (k+1)-th largest router logit is below 1e-3, and, when a drop
  threshold tau is set, while any of its renormalised top-k weights lies
  within 1e-4 of tau. This keeps the integer decisions of routing (which
  experts, which slots dropped) away from floating-point boundaries, so that
  the fp64 oracle and the fp32 GPU arithmetic must agree on them exactly.
  The logits and weights computed for this filter decide only *whether* to
  re-draw; they are never returned or compared against.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoegen.so")
_lib = None

# Tensor ids used as the second Philox key word.
TID_X, TID_WR, TID_W1, TID_W2, TID_W1S, TID_W2S, TID_PERM = 1, 2, 3, 4, 5, 6, 7

GAP_MIN = 1e-3       # minimum k-th / (k+1)-th logit gap
DROP_MARGIN = 1e-4   # minimum |w - tau| for every kept-candidate weight
MAX_ATTEMPTS = 256

# Workloads. ``seed`` fixes every array of a workload.
CONFIGS = {
    # Tiny fp32 layer, plus the parity-sized cases.
    "tiny": dict(T=64, H=64, F=128, E=4, k=2, Fs=0, drop=0.0, zipf=0.0, dtype="f32", seed=1001),
    # Decode: Qwen3-30B-A3B-like expert shapes (128 experts, top-8), 32 tokens.
    "decode": dict(T=32, H=2048, F=768, E=128, k=8, Fs=0, drop=0.0, zipf=0.0, dtype="bf16", seed=1002),
    # Prefill: same architecture, 8192 tokens (65,536 assignments).
    "prefill": dict(T=8192, H=2048, F=768, E=128, k=8, Fs=0, drop=0.0, zipf=0.0, dtype="bf16", seed=1003),
    # Mixtral-like 8 experts top-2 plus one always-on shared expert.
    "mixtral_shared": dict(T=4096, H=4096, F=14336, E=8, k=2, Fs=14336, drop=0.0, zipf=0.0, dtype="bf16",
                           seed=1004),
    # Skewed load: 64 experts top-2, Zipf(1.2) router bias, drop of weights < 0.05.
    "skew": dict(T=2048, H=5120, F=14336, E=64, k=2, Fs=0, drop=0.05, zipf=1.2, dtype="bf16", seed=1005),
}
CONFIG_ORDER = ["tiny", "decode", "prefill", "mixtral_shared", "skew"]


def lib_path() -> str:
    return _LIB_PATH


def build(force: bool = True) -> str:
    """Compile ``philox_normal.c`` into ``libmoegen.so`` with gcc and OpenMP."""
    import subprocess

    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        # separate libm sin and cos calls (no merged sincos): the deviates keep the same bits as every earlier build
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-fno-builtin-sin", "-fno-builtin-cos",
               os.path.join(_HERE, "philox_normal.c"), "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        u32, u64, dbl, vp = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        for name in ("moegen_normal_f64", "moegen_normal_f32", "moegen_normal_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [u32, u32, u32, u64, u64, dbl, vp]
            fn.restype = None
        lib.moegen_philox_raw.argtypes = [vp, vp, vp]
        lib.moegen_philox_raw.restype = None
        lib.moegen_philox_blocks.argtypes = [u32, u32, u32, u64, u64, vp]
        lib.moegen_philox_blocks.restype = None
        _lib = lib
    return _lib


def philox4x32_10(ctr, key) -> np.ndarray:
    """Raw Philox4x32-10 block (for the published known-answer vectors)."""
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    o = np.zeros(4, dtype=np.uint32)
    _load().moegen_philox_raw(c.ctypes.data, k.ctypes.data, o.ctypes.data)
    return o


def normal(seed: int, tid: int, n: int, std: float, dtype: str, attempt: int = 0, offset: int = 0) -> np.ndarray:
    """Elements [offset, offset+n) of stream (seed, tid, attempt), scaled by std and rounded.

    dtype: "f64" (unrounded), "f32", or "bf16" (returned as uint16 bit patterns).
    """
    lib = _load()
    if dtype == "f64":
        out = np.empty(n, dtype=np.float64)
        lib.moegen_normal_f64(seed, tid, attempt, offset, n, std, out.ctypes.data)
    elif dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        lib.moegen_normal_f32(seed, tid, attempt, offset, n, std, out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        lib.moegen_normal_bf16(seed, tid, attempt, offset, n, std, out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


_BF16_F64 = None


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (fp32, or bf16 bits) -> exact float64 values."""
    global _BF16_F64
    if dtype == "bf16":
        if _BF16_F64 is None:
            with np.errstate(invalid="ignore"):
                _BF16_F64 = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
        return _BF16_F64[np.asarray(a, dtype=np.uint16)]
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def zipf_probs(E: int, s: float) -> np.ndarray:
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    return p / p.sum()


@dataclasses.dataclass
class MoEInputs:
    """All arrays of one workload, in storage precision (fp32, or bf16 bits as uint16)."""

    name: str
    T: int
    H: int
    F: int
    E: int
    k: int
    Fs: int
    drop: float
    dtype: str
    seed: int
    x: np.ndarray                 # [T,H]
    Wr: np.ndarray                # [H,E]
    bias: Optional[np.ndarray]    # [E] float32 or None
    attempts: np.ndarray          # [T] re-draw attempt used for each token row
    beta: float = 0.0             # fitted Zipf scale (skewed workload)

    # --- expert weights are drawn on demand, so a caller can stream them ----
    def _std1(self) -> float:
        return 1.0 / np.sqrt(self.H)

    def W1(self, e0: int = 0, e1: Optional[int] = None) -> np.ndarray:
        """W1[e0:e1] as [n,H,F] (row-major, storage dtype)."""
        e1 = self.E if e1 is None else e1
        n = (e1 - e0) * self.H * self.F
        a = normal(self.seed, TID_W1, n, 1.0 / np.sqrt(self.H), self.dtype, 0, e0 * self.H * self.F)
        return a.reshape(e1 - e0, self.H, self.F)

    def W2(self, e0: int = 0, e1: Optional[int] = None) -> np.ndarray:
        """W2[e0:e1] as [n,F,H]."""
        e1 = self.E if e1 is None else e1
        n = (e1 - e0) * self.F * self.H
        a = normal(self.seed, TID_W2, n, 1.0 / np.sqrt(self.F), self.dtype, 0, e0 * self.F * self.H)
        return a.reshape(e1 - e0, self.F, self.H)

    def W1s(self) -> Optional[np.ndarray]:
        if not self.Fs:
            return None
        return normal(self.seed, TID_W1S, self.H * self.Fs, 1.0 / np.sqrt(self.H), self.dtype).reshape(self.H, self.Fs)

    def W2s(self) -> Optional[np.ndarray]:
        if not self.Fs:
            return None
        return normal(self.seed, TID_W2S, self.Fs * self.H, 1.0 / np.sqrt(self.Fs), self.dtype).reshape(self.Fs, self.H)

    def f64(self, a: Optional[np.ndarray]) -> Optional[np.ndarray]:
        if a is None:
            return None
        if a.dtype == np.float32 and self.dtype == "bf16":
            return a.astype(np.float64)  # fp32 side arrays (bias)
        return to_f64(a, self.dtype)

    def bias_f64(self) -> np.ndarray:
        if self.bias is None:
            return np.zeros(self.E, dtype=np.float64)
        return self.bias.astype(np.float64)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def _draw_rows(seed, tid, rows, H, std, dtype, attempts) -> np.ndarray:
    """Rows ``rows`` of a [*,H] tensor, each at its own attempt number."""
    out = []
    for t, a in zip(rows, attempts):
        out.append(normal(seed, tid, H, std, dtype, int(a), int(t) * H))
    return np.stack(out) if out else np.zeros((0, H), dtype=np.uint16 if dtype == "bf16" else np.float32)


def _near_tie_rows(x64, Wr64, b64, k, drop) -> np.ndarray:
    """Indices of token rows that sit too close to a routing decision boundary.

    Input conditioning only (see the module docstring): the values computed
    here decide whether a row is re-drawn and are then discarded.
    """
    E = Wr64.shape[1]
    s = x64 @ Wr64 + b64[None, :]
    s = -np.sort(-s, axis=1)
    bad = np.zeros(s.shape[0], dtype=bool)
    if k < E:
        bad |= (s[:, k - 1] - s[:, k]) < GAP_MIN
    if drop > 0:
        top = s[:, :k]
        p = np.exp(top - top[:, :1])
        p /= p.sum(axis=1, keepdims=True)
        bad |= np.any(np.abs(p - drop) < DROP_MARGIN, axis=1)
    return np.nonzero(bad)[0]


def _hot_share(x64, Wr64, b64, k) -> float:
    s = x64 @ Wr64 + b64[None, :]
    sel = np.argsort(-s, axis=1, kind="stable")[:, :k]
    counts = np.bincount(sel.ravel(), minlength=Wr64.shape[1])
    return counts.max() / sel.size


def fit_zipf_beta(x64, Wr64, log_p, k, lo=0.0, hi=8.0, target=0.375, tol=0.0125, iters=60) -> float:
    """Bisection on beta so that the hottest expert's top-k share is target +- tol."""
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        sh = _hot_share(x64, Wr64, mid * log_p, k)
        if abs(sh - target) <= tol:
            return mid
        if sh < target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def make_inputs(name: str = "tiny", seed: Optional[int] = None, **over) -> MoEInputs:
    """Build the inputs of a named workload; keyword overrides change its shape (T, H, F, E, k, ...)."""
    cfg = dict(CONFIGS[name]) if name in CONFIGS else dict(CONFIGS["tiny"])
    cfg.update(over)
    if seed is not None:
        cfg["seed"] = seed
    T, H, F, E, k = cfg["T"], cfg["H"], cfg["F"], cfg["E"], cfg["k"]
    dt, sd = cfg["dtype"], cfg["seed"]
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")

    x = normal(sd, TID_X, T * H, 1.0, dt).reshape(T, H)
    Wr = normal(sd, TID_WR, H * E, 1.0 / np.sqrt(H), dt).reshape(H, E)
    x64, Wr64 = to_f64(x, dt), to_f64(Wr, dt)

    bias = None
    beta = 0.0
    if cfg.get("zipf", 0.0) > 0:
        keys = normal(sd, TID_PERM, E, 1.0, "f64")
        rank = np.argsort(np.argsort(keys, kind="stable"), kind="stable")  # pi(e), 0-based
        log_p = np.log(zipf_probs(E, cfg["zipf"]))[rank]
        beta = fit_zipf_beta(x64, Wr64, log_p, k)
        bias = (beta * log_p).astype(np.float32)
    b64 = bias.astype(np.float64) if bias is not None else np.zeros(E)

    attempts = np.zeros(T, dtype=np.int64)
    bad = _near_tie_rows(x64, Wr64, b64, k, cfg["drop"])
    while bad.size:
        attempts[bad] += 1
        if attempts.max() >= MAX_ATTEMPTS:
            raise RuntimeError("near-tie re-draw did not converge")
        rows = _draw_rows(sd, TID_X, bad, H, 1.0, dt, attempts[bad])
        x[bad] = rows
        x64[bad] = to_f64(rows, dt)
        sub = _near_tie_rows(x64[bad], Wr64, b64, k, cfg["drop"])
        bad = bad[sub]

    return MoEInputs(name=name, T=T, H=H, F=F, E=E, k=k, Fs=cfg.get("Fs", 0), drop=float(cfg["drop"]),
                     dtype=dt, seed=sd, x=x, Wr=Wr, bias=bias, attempts=attempts, beta=beta)


# ------------------------------------------------------------ device upload --
def storage_to_torch(a: np.ndarray, dtype: str):
    """Storage array -> CPU torch tensor (bf16 bits reinterpreted as torch.bfloat16)."""
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def to_device(I: MoEInputs, device="cuda", experts_per_chunk: Optional[int] = None, keep_host: bool = False) -> dict:
    """Copy every array of a workload to `device`; expert weights are drawn and copied in chunks.

    keep_host: also return the drawn expert weights in storage precision as ``W1_host`` [E,H,F] and
    ``W2_host`` [E,F,H] (numpy), so that a caller needing them on the host does not draw them again."""
    import torch

    tdt = torch.bfloat16 if I.dtype == "bf16" else torch.float32
    out = {"x": storage_to_torch(I.x, I.dtype).to(device), "Wr": storage_to_torch(I.Wr, I.dtype).to(device),
           "bias": torch.from_numpy(I.bias).to(device) if I.bias is not None else None}
    per_expert = I.H * I.F
    if experts_per_chunk is None:
        experts_per_chunk = max(1, (256 << 20) // max(1, per_expert))
    W1 = torch.empty((I.E, I.H, I.F), dtype=tdt, device=device)
    W2 = torch.empty((I.E, I.F, I.H), dtype=tdt, device=device)
    host = {"W1": [], "W2": []}
    for e0 in range(0, I.E, experts_per_chunk):
        e1 = min(I.E, e0 + experts_per_chunk)
        w1, w2 = I.W1(e0, e1), I.W2(e0, e1)
        W1[e0:e1].copy_(storage_to_torch(w1, I.dtype))
        W2[e0:e1].copy_(storage_to_torch(w2, I.dtype))
        if keep_host:
            host["W1"].append(w1)
            host["W2"].append(w2)
    out["W1"], out["W2"] = W1, W2
    if keep_host:
        out["W1_host"] = np.concatenate(host["W1"])
        out["W2_host"] = np.concatenate(host["W2"])
    out["W1s"] = storage_to_torch(I.W1s(), I.dtype).to(device) if I.Fs else None
    out["W2s"] = storage_to_torch(I.W2s(), I.dtype).to(device) if I.Fs else None
    return out
