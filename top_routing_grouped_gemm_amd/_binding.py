"""ctypes binding of ``libmoe.so`` (declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels.
torch supplies device memory and the stream. There is no CPU fallback: if the
library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loads torch's HIP runtime first, which libmoe.so then shares

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4

EXPORTS = ("moe_strerror", "moe_version", "moe_workspace_bytes", "moe_route_workspace_bytes",
           "moe_permute_workspace_bytes", "moe_ffn_workspace_bytes", "moe_route", "moe_permute", "moe_grouped_ffn",
           "moe_combine", "moe_forward", "moe_route_capacity_workspace_bytes", "moe_route_capacity",
           "moe_select_capacity_workspace_bytes", "moe_select_capacity", "moe_pad_dispatch",
           "moe_grouped_ffn_padded_workspace_bytes", "moe_grouped_ffn_padded", "moe_fp8_weight_bytes",
           "moe_quantize_fp8", "moe_grouped_ffn_fp8", "moe_forward_fp8", "moe_mxfp8_weight_bytes",
           "moe_mxfp8_scale_bytes", "moe_quantize_mxfp8", "moe_quantize_mxfp8_rows", "moe_mxfp8_workspace_bytes", "moe_grouped_ffn_mxfp8",
           "moe_grouped_ffn_mxfp8_workspace_bytes",
           "moe_forward_mxfp8", "moe_calibrate_mfma_bf16", "moe_calibrate_stream_read",
           "moe_forward_noalloc", "moe_grouped_ffn_fused", "moe_calibrate_gemm_kstep")


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} ({status})")


_lib = None


def load_library(path: Optional[str] = None):
    """Load libmoe.so and declare its signatures. Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it first (python -m top_routing_grouped_gemm_amd.build)")
    lib = ctypes.CDLL(p)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.moe_strerror.argtypes = [i32]
    lib.moe_strerror.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_version.restype = ctypes.c_char_p
    lib.moe_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.moe_workspace_bytes.restype = sz
    lib.moe_route_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.moe_route_workspace_bytes.restype = sz
    lib.moe_permute_workspace_bytes.argtypes = [i32, i32, i32]
    lib.moe_permute_workspace_bytes.restype = sz
    lib.moe_ffn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.moe_ffn_workspace_bytes.restype = sz
    lib.moe_route.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, vp, vp, sz, vp]
    lib.moe_route.restype = i32
    lib.moe_route_capacity_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.moe_route_capacity_workspace_bytes.restype = sz
    lib.moe_route_capacity.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, ctypes.c_double, i32, vp, vp, vp, sz, vp]
    lib.moe_route_capacity.restype = i32
    lib.moe_select_capacity_workspace_bytes.argtypes = [i32, i32]
    lib.moe_select_capacity_workspace_bytes.restype = sz
    lib.moe_select_capacity.argtypes = [vp, i32, i32, i32, f32, i32, vp, vp, vp, sz, vp]
    lib.moe_select_capacity.restype = i32
    lib.moe_pad_dispatch.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.moe_pad_dispatch.restype = i32
    lib.moe_grouped_ffn_padded_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.moe_grouped_ffn_padded_workspace_bytes.restype = sz
    lib.moe_grouped_ffn_padded.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, sz, vp]
    lib.moe_grouped_ffn_padded.restype = i32
    lib.moe_permute.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_permute.restype = i32
    lib.moe_grouped_ffn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, i32, vp, vp, sz,
                                    vp]
    lib.moe_grouped_ffn.restype = i32
    lib.moe_grouped_ffn_fused.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.moe_grouped_ffn_fused.restype = i32
    lib.moe_combine.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp]
    lib.moe_combine.restype = i32
    lib.moe_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp, i32, vp, vp,
                                vp, vp, vp, sz, vp]
    lib.moe_forward.restype = i32
    lib.moe_fp8_weight_bytes.argtypes = [i32, i32, i32]
    lib.moe_fp8_weight_bytes.restype = sz
    lib.moe_quantize_fp8.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
    lib.moe_quantize_fp8.restype = i32
    lib.moe_grouped_ffn_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, sz, vp]
    lib.moe_grouped_ffn_fp8.restype = i32
    lib.moe_forward_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, i32, vp, vp, vp, vp,
                                    vp, sz, vp]
    lib.moe_forward_fp8.restype = i32
    lib.moe_mxfp8_weight_bytes.argtypes = [i32, i32, i32]
    lib.moe_mxfp8_weight_bytes.restype = sz
    lib.moe_mxfp8_scale_bytes.argtypes = [i32, i32, i32]
    lib.moe_mxfp8_scale_bytes.restype = sz
    lib.moe_quantize_mxfp8.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
    lib.moe_quantize_mxfp8.restype = i32
    lib.moe_quantize_mxfp8_rows.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.moe_quantize_mxfp8_rows.restype = i32
    lib.moe_mxfp8_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.moe_mxfp8_workspace_bytes.restype = sz
    lib.moe_grouped_ffn_mxfp8_workspace_bytes.argtypes = [i32, i32, i32]
    lib.moe_grouped_ffn_mxfp8_workspace_bytes.restype = sz
    lib.moe_grouped_ffn_mxfp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.moe_grouped_ffn_mxfp8.restype = i32
    lib.moe_forward_mxfp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, i32, vp, vp, vp,
                                      vp, vp, sz, vp]
    lib.moe_forward_mxfp8.restype = i32
    lib.moe_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp, i32,
                                        vp, vp, vp, vp, vp]
    lib.moe_forward_noalloc.restype = i32
    lib.moe_calibrate_mfma_bf16.argtypes = [i32, i32, i32, i32, vp, vp]
    lib.moe_calibrate_mfma_bf16.restype = i32
    lib.moe_calibrate_stream_read.argtypes = [vp, sz, i32, vp, vp]
    lib.moe_calibrate_stream_read.restype = i32
    lib.moe_calibrate_gemm_kstep.argtypes = [vp, sz, i32, i32, i32, vp, vp]
    lib.moe_calibrate_gemm_kstep.restype = i32
    if path is None:
        _lib = lib
    return lib


def strerror(status: int) -> str:
    return load_library().moe_strerror(int(status)).decode()


def version() -> str:
    return load_library().moe_version().decode()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _arg(t, name: str, shape=None, dtype=None, device=None, optional: bool = False):
    """Validate one tensor argument before any pointer reaches the library: a kernel given a short buffer or the
    wrong element type would read or write out of bounds. ``shape`` is a tuple (None entries match any size),
    ``dtype`` a torch dtype or a tuple of them; ``device`` the device every tensor of the call must share."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if dtype is not None:
        allowed = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in allowed:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in allowed)}")
    if shape is not None:
        ok = t.dim() == len(shape) and all(s is None or int(a) == int(s) for a, s in zip(t.shape, shape))
        if not ok:
            want = "[" + ", ".join("*" if s is None else str(int(s)) for s in shape) + "]"
            raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device} like the other tensors")
    # placement on the GPU and contiguity are checked when the pointer is taken (_ptr)


def _ws_arg(ws, device):
    """A caller workspace: a contiguous uint8 tensor on the call's device (its byte count is checked in C)."""
    _arg(ws, "ws", None, torch.uint8, device, optional=True)


_FLOAT = (torch.bfloat16, torch.float32)


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def moe_workspace_bytes(T, H, F, E, k, Fs=0, dtype=torch.bfloat16) -> int:
    dt = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
    return int(load_library().moe_workspace_bytes(T, H, F, E, k, Fs, dt))


def moe_route_workspace_bytes(T, H, E, dtype=torch.bfloat16) -> int:
    dt = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
    return int(load_library().moe_route_workspace_bytes(T, H, E, dt))


def moe_permute_workspace_bytes(T, E, k) -> int:
    return int(load_library().moe_permute_workspace_bytes(T, E, k))


def moe_ffn_workspace_bytes(T, F, E, k, Fs=0, dtype=torch.bfloat16) -> int:
    dt = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
    return int(load_library().moe_ffn_workspace_bytes(T, F, E, k, Fs, dt))


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def moe_route(x, Wr, bias, k: int, drop_thresh: float = 0.0, topk_ids=None, topk_w=None, ws=None, stream=None):
    """Router logits, top-k, softmax weights (+ drop). Returns (topk_ids [T,k] int32, topk_w [T,k] fp32)."""
    _arg(x, "x", (None, None), _FLOAT)
    T, H = x.shape
    dev = x.device
    _arg(x, "x", device=dev)
    _arg(Wr, "Wr", (H, None), x.dtype, dev)
    E = Wr.shape[1]
    _arg(bias, "bias", (E,), torch.float32, dev, optional=True)
    topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_ids is None else topk_ids
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    _arg(topk_ids, "topk_ids", (T, k), torch.int32, dev)
    _arg(topk_w, "topk_w", (T, k), torch.float32, dev)
    _ws_arg(ws, dev)
    need = moe_route_workspace_bytes(T, H, E, x.dtype)
    if ws is None and need > 0:
        ws = _ws(need, dev)
    st = load_library().moe_route(_ptr(x), _ptr(Wr), _ptr(bias), T, H, E, k, float(drop_thresh), _dt(x),
                                  _ptr(topk_ids), _ptr(topk_w), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(stream))
    _check(st, "moe_route")
    return topk_ids, topk_w


def moe_route_capacity(x, Wr, bias, k: int, drop_thresh: float = 0.0, cap_factor: float = 1.2, topk_ids=None,
                       topk_w=None, ws=None, stream=None):
    """Router logits, capacity-limited top-k, softmax weights (+ drop). Returns (topk_ids, topk_w)."""
    _arg(x, "x", (None, None), _FLOAT)
    T, H = x.shape
    dev = x.device
    _arg(x, "x", device=dev)
    _arg(Wr, "Wr", (H, None), x.dtype, dev)
    E = Wr.shape[1]
    _arg(bias, "bias", (E,), torch.float32, dev, optional=True)
    topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_ids is None else topk_ids
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    _arg(topk_ids, "topk_ids", (T, k), torch.int32, dev)
    _arg(topk_w, "topk_w", (T, k), torch.float32, dev)
    _ws_arg(ws, dev)
    dt = _dt(x)
    ws = _ws(load_library().moe_route_capacity_workspace_bytes(T, H, E, dt), dev) if ws is None else ws
    st = load_library().moe_route_capacity(_ptr(x), _ptr(Wr), _ptr(bias), T, H, E, k, float(drop_thresh),
                                           float(cap_factor), dt, _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ws.numel(),
                                           _stream(stream))
    _check(st, "moe_route_capacity")
    return topk_ids, topk_w


def moe_select_capacity(logits, k: int, cap: int, drop_thresh: float = 0.0, topk_ids=None, topk_w=None, ws=None,
                        stream=None):
    """Capacity-limited top-k + weights on fp32 logits [T,E]. Returns (topk_ids, topk_w)."""
    _arg(logits, "logits", (None, None), torch.float32)
    T, E = logits.shape
    dev = logits.device
    topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_ids is None else topk_ids
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    _arg(topk_ids, "topk_ids", (T, k), torch.int32, dev)
    _arg(topk_w, "topk_w", (T, k), torch.float32, dev)
    _ws_arg(ws, dev)
    ws = _ws(load_library().moe_select_capacity_workspace_bytes(T, E), dev) if ws is None else ws
    st = load_library().moe_select_capacity(_ptr(logits), T, E, k, float(drop_thresh), int(cap), _ptr(topk_ids),
                                            _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_select_capacity")
    return topk_ids, topk_w


def moe_permute(x, topk_ids, topk_w, E: int, x_perm=None, expert_offsets=None, row_token=None, inv=None, ws=None,
                stream=None):
    """Dispatch. Returns (x_perm [T*k,H], expert_offsets [E+1], row_token [T*k], inv [T,k])."""
    _arg(x, "x", (None, None), _FLOAT)
    T, H = x.shape
    dev = x.device
    _arg(topk_ids, "topk_ids", (T, None), torch.int32, dev)
    k = topk_ids.shape[1]
    _arg(topk_w, "topk_w", (T, k), torch.float32, dev)
    x_perm = torch.empty((T * k, H), dtype=x.dtype, device=dev) if x_perm is None else x_perm
    expert_offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if expert_offsets is None else expert_offsets
    row_token = torch.empty(T * k, dtype=torch.int32, device=dev) if row_token is None else row_token
    inv = torch.empty((T, k), dtype=torch.int32, device=dev) if inv is None else inv
    _arg(x_perm, "x_perm", (T * k, H), x.dtype, dev)
    _arg(expert_offsets, "expert_offsets", (E + 1,), torch.int32, dev)
    _arg(row_token, "row_token", (T * k,), torch.int32, dev)
    _arg(inv, "inv", (T, k), torch.int32, dev)
    _ws_arg(ws, dev)
    need = moe_permute_workspace_bytes(T, E, k)
    ws = _ws(need, dev) if ws is None else ws
    st = load_library().moe_permute(_ptr(x), _ptr(topk_ids), _ptr(topk_w), T, H, E, k, _dt(x), _ptr(x_perm),
                                    _ptr(expert_offsets), _ptr(row_token), _ptr(inv), _ptr(ws), ws.numel(),
                                    _stream(stream))
    _check(st, "moe_permute")
    return x_perm, expert_offsets, row_token, inv


def moe_grouped_ffn(x_perm, expert_offsets, W1, W2, T: int, k: int, y_perm=None, x=None, W1s=None, W2s=None,
                    y_shared=None, ws=None, stream=None):
    """Grouped FFN over all experts (+ shared). Returns (y_perm [T*k,H] fp32, y_shared [T,H] fp32 or None)."""
    _arg(x_perm, "x_perm", (T * k, None), _FLOAT)
    dt, dev = x_perm.dtype, x_perm.device
    _arg(W1, "W1", (None, x_perm.shape[1], None), dt, dev)
    E, H, F = W1.shape
    _arg(W2, "W2", (E, F, H), dt, dev)
    _arg(expert_offsets, "expert_offsets", (E + 1,), torch.int32, dev)
    if (W1s is None) != (W2s is None):
        raise ValueError("the shared expert needs both W1s and W2s")
    Fs = W1s.shape[1] if W1s is not None else 0
    _arg(W1s, "W1s", (H, None), dt, dev, optional=True)
    _arg(W2s, "W2s", (Fs, H), dt, dev, optional=W1s is None)
    _arg(x, "x", (T, H), dt, dev, optional=W1s is None)
    y_perm = torch.empty((T * k, H), dtype=torch.float32, device=dev) if y_perm is None else y_perm
    if W1s is not None and y_shared is None:
        y_shared = torch.empty((T, H), dtype=torch.float32, device=dev)
    _arg(y_perm, "y_perm", (T * k, H), torch.float32, dev)
    _arg(y_shared, "y_shared", (T, H), torch.float32, dev, optional=W1s is None)
    _ws_arg(ws, dev)
    need = moe_ffn_workspace_bytes(T, F, E, k, Fs, x_perm.dtype)
    ws = _ws(need, dev) if ws is None else ws
    st = load_library().moe_grouped_ffn(_ptr(x_perm), _ptr(expert_offsets), _ptr(W1), _ptr(W2), T, H, F, E, k,
                                        _dt(x_perm), _ptr(y_perm), _ptr(x), _ptr(W1s), _ptr(W2s), Fs, _ptr(y_shared),
                                        _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_grouped_ffn")
    return y_perm, y_shared


def moe_grouped_ffn_fused(x_perm, expert_offsets, W1, W2, T: int, k: int, y_perm=None, stream=None):
    """Grouped FFN in one launch with h kept on chip (bf16, F % 256 == 0, F <= 768, H % 256 == 0).
    Returns y_perm [T*k,H] fp32; other shapes raise MoEError (MOE_ERR_UNSUPPORTED)."""
    _arg(x_perm, "x_perm", (T * k, None), _FLOAT)
    dt, dev = x_perm.dtype, x_perm.device
    _arg(W1, "W1", (None, x_perm.shape[1], None), dt, dev)
    E, H, F = W1.shape
    _arg(W2, "W2", (E, F, H), dt, dev)
    _arg(expert_offsets, "expert_offsets", (E + 1,), torch.int32, dev)
    y_perm = torch.empty((T * k, H), dtype=torch.float32, device=dev) if y_perm is None else y_perm
    _arg(y_perm, "y_perm", (T * k, H), torch.float32, dev)
    st = load_library().moe_grouped_ffn_fused(_ptr(x_perm), _ptr(expert_offsets), _ptr(W1), _ptr(W2), T, H, F, E, k,
                                              _dt(x_perm), _ptr(y_perm), _stream(stream))
    _check(st, "moe_grouped_ffn_fused")
    return y_perm


def moe_pad_dispatch(x, topk_ids, expert_offsets, row_token, inv, E: int, C: int, x_pad=None, inv_pad=None,
                     stream=None):
    """Padded layout from moe_permute's maps. Returns (x_pad [E*C,H], inv_pad [T,k])."""
    _arg(x, "x", (None, None), _FLOAT)
    T, H = x.shape
    dev = x.device
    _arg(topk_ids, "topk_ids", (T, None), torch.int32, dev)
    k = topk_ids.shape[1]
    _arg(expert_offsets, "expert_offsets", (E + 1,), torch.int32, dev)
    _arg(row_token, "row_token", (T * k,), torch.int32, dev)
    _arg(inv, "inv", (T, k), torch.int32, dev)
    x_pad = torch.empty((E * C, H), dtype=x.dtype, device=dev) if x_pad is None else x_pad
    inv_pad = torch.empty((T, k), dtype=torch.int32, device=dev) if inv_pad is None else inv_pad
    _arg(x_pad, "x_pad", (E * C, H), x.dtype, dev)
    _arg(inv_pad, "inv_pad", (T, k), torch.int32, dev)
    st = load_library().moe_pad_dispatch(_ptr(x), _ptr(topk_ids), _ptr(expert_offsets), _ptr(row_token), _ptr(inv),
                                         T, H, E, k, C, _dt(x), _ptr(x_pad), _ptr(inv_pad), _stream(stream))
    _check(st, "moe_pad_dispatch")
    return x_pad, inv_pad


def moe_grouped_ffn_padded(x_pad, W1, W2, C: int, y_pad=None, ws=None, stream=None):
    """Every expert's FFN over its C padded rows. Returns y_pad [E*C,H] fp32."""
    _arg(x_pad, "x_pad", (None, None), _FLOAT)
    dt, dev = x_pad.dtype, x_pad.device
    _arg(W1, "W1", (None, x_pad.shape[1], None), dt, dev)
    E, H, F = W1.shape
    _arg(x_pad, "x_pad", (E * C, H))
    _arg(W2, "W2", (E, F, H), dt, dev)
    y_pad = torch.empty((E * C, H), dtype=torch.float32, device=dev) if y_pad is None else y_pad
    _arg(y_pad, "y_pad", (E * C, H), torch.float32, dev)
    _ws_arg(ws, dev)
    need = load_library().moe_grouped_ffn_padded_workspace_bytes(E, C, H, F, _dt(x_pad))
    ws = _ws(need, dev) if ws is None else ws
    st = load_library().moe_grouped_ffn_padded(_ptr(x_pad), _ptr(W1), _ptr(W2), E, C, H, F, _dt(x_pad), _ptr(y_pad),
                                               _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_grouped_ffn_padded")
    return y_pad


def moe_combine(y_perm, inv, topk_w, y_shared=None, out_dtype=torch.float32, y=None, stream=None):
    """Unpermute + weighted sum. Returns y [T,H] in out_dtype."""
    # inv's entries must index rows of y_perm (moe_permute / moe_pad_dispatch write such maps); they stay on the
    # device and are not checked here
    _arg(y_perm, "y_perm", (None, None), torch.float32)
    dev = y_perm.device
    _arg(inv, "inv", (None, None), torch.int32, dev)
    T, k = inv.shape
    H = y_perm.shape[1]
    _arg(topk_w, "topk_w", (T, k), torch.float32, dev)
    _arg(y_shared, "y_shared", (T, H), torch.float32, dev, optional=True)
    y = torch.empty((T, H), dtype=out_dtype, device=dev) if y is None else y
    _arg(y, "y", (T, H), _FLOAT, dev)
    st = load_library().moe_combine(_ptr(y_perm), _ptr(inv), _ptr(topk_w), _ptr(y_shared), T, H, k, _dt(y), _ptr(y),
                                    _stream(stream))
    _check(st, "moe_combine")
    return y


def moe_forward(x, Wr, bias, W1, W2, k: int, drop_thresh: float = 0.0, W1s=None, W2s=None, out_dtype=torch.float32,
                y=None, topk_ids=None, topk_w=None, expert_offsets=None, inv=None, ws=None, stream=None):
    """The whole layer. Returns y [T,H]; the optional debug tensors are filled when given."""
    _arg(x, "x", (None, None), _FLOAT)
    T, H = x.shape
    dt, dev = x.dtype, x.device
    _arg(Wr, "Wr", (H, None), dt, dev)
    E = Wr.shape[1]
    _arg(bias, "bias", (E,), torch.float32, dev, optional=True)
    _arg(W1, "W1", (E, H, None), dt, dev)
    F = W1.shape[2]
    _arg(W2, "W2", (E, F, H), dt, dev)
    if (W1s is None) != (W2s is None):
        raise ValueError("the shared expert needs both W1s and W2s")
    Fs = W1s.shape[1] if W1s is not None else 0
    _arg(W1s, "W1s", (H, None), dt, dev, optional=True)
    _arg(W2s, "W2s", (Fs, H), dt, dev, optional=W1s is None)
    y = torch.empty((T, H), dtype=out_dtype, device=dev) if y is None else y
    _arg(y, "y", (T, H), _FLOAT, dev)
    _forward_debug_args(T, E, k, topk_ids, topk_w, expert_offsets, inv, dev)
    _ws_arg(ws, dev)
    need = moe_workspace_bytes(T, H, F, E, k, Fs, x.dtype)
    ws = _ws(need, dev) if ws is None else ws
    st = load_library().moe_forward(_ptr(x), _ptr(Wr), _ptr(bias), _ptr(W1), _ptr(W2), _ptr(W1s), _ptr(W2s), Fs, T, H,
                                    F, E, k, float(drop_thresh), _dt(x), _ptr(y), _dt(y), _ptr(topk_ids),
                                    _ptr(topk_w), _ptr(expert_offsets), _ptr(inv), _ptr(ws), ws.numel(),
                                    _stream(stream))
    _check(st, "moe_forward")
    return y


def _forward_debug_args(T, E, k, topk_ids, topk_w, expert_offsets, inv, dev):
    _arg(topk_ids, "topk_ids", (T, k), torch.int32, dev, optional=True)
    _arg(topk_w, "topk_w", (T, k), torch.float32, dev, optional=True)
    _arg(expert_offsets, "expert_offsets", (E + 1,), torch.int32, dev, optional=True)
    _arg(inv, "inv", (T, k), torch.int32, dev, optional=True)


def _fp8_weights(W1q, W1_scale, W2q, W2_scale, E, H, F, dev):
    """The tiled fp8 codes and per-column scales of both expert matrices, as moe_quantize_fp8 returns them."""
    _arg(W1q, "W1q", (moe_fp8_weight_bytes(E, H, F),), torch.uint8, dev)
    _arg(W1_scale, "W1_scale", (E, F), torch.float32, dev)
    _arg(W2q, "W2q", (moe_fp8_weight_bytes(E, F, H),), torch.uint8, dev)
    _arg(W2_scale, "W2_scale", (E, H), torch.float32, dev)


def _mx_weights(W1q, W1_scale, W2q, W2_scale, E, H, F, dev):
    """The MX code tiles and scale bytes of both expert matrices, as moe_quantize_mxfp8 returns them."""
    lib = load_library()
    _arg(W1q, "W1q", (int(lib.moe_mxfp8_weight_bytes(E, H, F)),), torch.uint8, dev)
    _arg(W1_scale, "W1_scale", (int(lib.moe_mxfp8_scale_bytes(E, H, F)),), torch.uint8, dev)
    _arg(W2q, "W2q", (int(lib.moe_mxfp8_weight_bytes(E, F, H)),), torch.uint8, dev)
    _arg(W2_scale, "W2_scale", (int(lib.moe_mxfp8_scale_bytes(E, F, H)),), torch.uint8, dev)


def moe_forward_noalloc(x, Wr, bias, W1, W2, k: int, drop_thresh: float = 0.0, W1s=None, W2s=None,
                        out_dtype=torch.float32, y=None, topk_ids=None, topk_w=None, expert_offsets=None, inv=None,
                        stream=None):
    """moe_forward without a workspace: the intermediate buffers live in the library's static per-GPU scratch
    array (see include/moe.h for its size limit; calls that overlap on one GPU race on it). Returns y [T,H]."""
    _arg(x, "x", (None, None), _FLOAT)
    T, H = x.shape
    dt, dev = x.dtype, x.device
    _arg(Wr, "Wr", (H, None), dt, dev)
    E = Wr.shape[1]
    _arg(bias, "bias", (E,), torch.float32, dev, optional=True)
    _arg(W1, "W1", (E, H, None), dt, dev)
    F = W1.shape[2]
    _arg(W2, "W2", (E, F, H), dt, dev)
    if (W1s is None) != (W2s is None):
        raise ValueError("the shared expert needs both W1s and W2s")
    Fs = W1s.shape[1] if W1s is not None else 0
    _arg(W1s, "W1s", (H, None), dt, dev, optional=True)
    _arg(W2s, "W2s", (Fs, H), dt, dev, optional=W1s is None)
    y = torch.empty((T, H), dtype=out_dtype, device=dev) if y is None else y
    _arg(y, "y", (T, H), _FLOAT, dev)
    _forward_debug_args(T, E, k, topk_ids, topk_w, expert_offsets, inv, dev)
    st = load_library().moe_forward_noalloc(_ptr(x), _ptr(Wr), _ptr(bias), _ptr(W1), _ptr(W2), _ptr(W1s), _ptr(W2s),
                                            Fs, T, H, F, E, k, float(drop_thresh), _dt(x), _ptr(y), _dt(y),
                                            _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets), _ptr(inv),
                                            _stream(stream))
    _check(st, "moe_forward_noalloc")
    return y


def moe_fp8_weight_bytes(E: int, K: int, N: int) -> int:
    return int(load_library().moe_fp8_weight_bytes(E, K, N))


def moe_quantize_fp8(W, Wq=None, scales=None, stream=None):
    """fp8 e4m3 codes of W [E,K,N] (bf16 or fp32) in the tiled layout of
    include/moe.h, with per-expert, per-column fp32 scales.
    Returns (Wq uint8 [moe_fp8_weight_bytes(E,K,N)], scales [E,N] fp32)."""
    _arg(W, "W", (None, None, None), _FLOAT)
    E, K, N = W.shape
    dev = W.device
    nbytes = moe_fp8_weight_bytes(E, K, N)
    if nbytes == 0:
        _check(MOE_ERR_UNSUPPORTED, "moe_fp8_weight_bytes")
    Wq = torch.empty(nbytes, dtype=torch.uint8, device=dev) if Wq is None else Wq
    scales = torch.empty((E, N), dtype=torch.float32, device=dev) if scales is None else scales
    _arg(Wq, "Wq", (nbytes,), torch.uint8, dev)
    _arg(scales, "scales", (E, N), torch.float32, dev)
    st = load_library().moe_quantize_fp8(_ptr(W), E, K, N, _dt(W), _ptr(Wq), _ptr(scales), _stream(stream))
    _check(st, "moe_quantize_fp8")
    return Wq, scales


def moe_grouped_ffn_fp8(x_perm, expert_offsets, W1q, W1_scale, W2q, W2_scale, T: int, k: int, y_perm=None, ws=None,
                        stream=None):
    """Grouped FFN on fp8 experts (scales W1_scale [E,F], W2_scale [E,H]). Returns y_perm [T*k,H] fp32."""
    _arg(x_perm, "x_perm", (T * k, None), torch.bfloat16)
    dev = x_perm.device
    H = x_perm.shape[1]
    _arg(W1_scale, "W1_scale", (None, None), torch.float32, dev)
    E, F = W1_scale.shape
    _fp8_weights(W1q, W1_scale, W2q, W2_scale, E, H, F, dev)
    _arg(expert_offsets, "expert_offsets", (E + 1,), torch.int32, dev)
    y_perm = torch.empty((T * k, H), dtype=torch.float32, device=dev) if y_perm is None else y_perm
    _arg(y_perm, "y_perm", (T * k, H), torch.float32, dev)
    _ws_arg(ws, dev)
    need = moe_ffn_workspace_bytes(T, F, E, k, 0, torch.bfloat16)
    ws = _ws(need, dev) if ws is None else ws
    st = load_library().moe_grouped_ffn_fp8(_ptr(x_perm), _ptr(expert_offsets), _ptr(W1q), _ptr(W1_scale), _ptr(W2q),
                                            _ptr(W2_scale), T, H, F, E, k, _ptr(y_perm), _ptr(ws), ws.numel(),
                                            _stream(stream))
    _check(st, "moe_grouped_ffn_fp8")
    return y_perm


def moe_forward_fp8(x, Wr, bias, W1q, W1_scale, W2q, W2_scale, k: int, drop_thresh: float = 0.0,
                    out_dtype=torch.float32, y=None, topk_ids=None, topk_w=None, expert_offsets=None, inv=None,
                    ws=None, stream=None):
    """The whole layer with fp8 experts (x, Wr bf16). Returns y [T,H]."""
    _arg(x, "x", (None, None), torch.bfloat16)
    T, H = x.shape
    dev = x.device
    _arg(W1_scale, "W1_scale", (None, None), torch.float32, dev)
    E, F = W1_scale.shape
    _arg(Wr, "Wr", (H, E), torch.bfloat16, dev)
    _arg(bias, "bias", (E,), torch.float32, dev, optional=True)
    _fp8_weights(W1q, W1_scale, W2q, W2_scale, E, H, F, dev)
    y = torch.empty((T, H), dtype=out_dtype, device=dev) if y is None else y
    _arg(y, "y", (T, H), _FLOAT, dev)
    _forward_debug_args(T, E, k, topk_ids, topk_w, expert_offsets, inv, dev)
    _ws_arg(ws, dev)
    need = moe_workspace_bytes(T, H, F, E, k, 0, torch.bfloat16)
    ws = _ws(need, dev) if ws is None else ws
    st = load_library().moe_forward_fp8(_ptr(x), _ptr(Wr), _ptr(bias), _ptr(W1q), _ptr(W1_scale), _ptr(W2q),
                                        _ptr(W2_scale), T, H, F, E, k, float(drop_thresh), _ptr(y), _dt(y),
                                        _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets), _ptr(inv), _ptr(ws),
                                        ws.numel(), _stream(stream))
    _check(st, "moe_forward_fp8")
    return y


def moe_quantize_mxfp8(W, Wq=None, W_scale=None, stream=None):
    """MX fp8 codes of W [E,K,N] (blocks of 32 along K) in the tiled layout of
    include/moe.h, and their scale bytes. Returns (Wq uint8, W_scale uint8)."""
    _arg(W, "W", (None, None, None), _FLOAT)
    E, K, N = W.shape
    lib = load_library()
    nq, ns = int(lib.moe_mxfp8_weight_bytes(E, K, N)), int(lib.moe_mxfp8_scale_bytes(E, K, N))
    if nq == 0:
        _check(MOE_ERR_UNSUPPORTED, "moe_mxfp8_weight_bytes")
    Wq = torch.empty(nq, dtype=torch.uint8, device=W.device) if Wq is None else Wq
    W_scale = torch.empty(ns, dtype=torch.uint8, device=W.device) if W_scale is None else W_scale
    _arg(Wq, "Wq", (nq,), torch.uint8, W.device)
    _arg(W_scale, "W_scale", (ns,), torch.uint8, W.device)
    st = lib.moe_quantize_mxfp8(_ptr(W), E, K, N, _dt(W), _ptr(Wq), _ptr(W_scale), _stream(stream))
    _check(st, "moe_quantize_mxfp8")
    return Wq, W_scale


def moe_quantize_mxfp8_rows(x, xq=None, x_scale=None, stream=None):
    """MX fp8 codes of the rows of x [T,H] (blocks of 32 along H): xq [T,H] uint8 and the
    scale bytes [H/128, T, 4] uint8."""
    _arg(x, "x", (None, None), _FLOAT)
    T, H = x.shape
    xq = torch.empty((T, H), dtype=torch.uint8, device=x.device) if xq is None else xq
    x_scale = torch.empty((H // 128, T, 4), dtype=torch.uint8, device=x.device) if x_scale is None else x_scale
    _arg(xq, "xq", (T, H), torch.uint8, x.device)
    _arg(x_scale, "x_scale", (H // 128, T, 4), torch.uint8, x.device)
    st = load_library().moe_quantize_mxfp8_rows(_ptr(x), T, H, _dt(x), _ptr(xq), _ptr(x_scale), _stream(stream))
    _check(st, "moe_quantize_mxfp8_rows")
    return xq, x_scale


def moe_forward_mxfp8(x, Wr, bias, W1q, W1_scale, W2q, W2_scale, F: int, k: int, drop_thresh: float = 0.0,
                      E: Optional[int] = None, out_dtype=torch.float32, y=None, topk_ids=None, topk_w=None,
                      expert_offsets=None, inv=None, ws=None, stream=None):
    """The whole layer with MX fp8 experts (x, Wr bf16). Returns y [T,H]."""
    _arg(x, "x", (None, None), torch.bfloat16)
    T, H = x.shape
    dev = x.device
    _arg(Wr, "Wr", (H, None), torch.bfloat16, dev)
    E = Wr.shape[1] if E is None else E
    _arg(Wr, "Wr", (H, E))
    _arg(bias, "bias", (E,), torch.float32, dev, optional=True)
    _mx_weights(W1q, W1_scale, W2q, W2_scale, E, H, F, dev)
    lib = load_library()
    y = torch.empty((T, H), dtype=out_dtype, device=dev) if y is None else y
    _arg(y, "y", (T, H), _FLOAT, dev)
    _forward_debug_args(T, E, k, topk_ids, topk_w, expert_offsets, inv, dev)
    _ws_arg(ws, dev)
    need = int(lib.moe_mxfp8_workspace_bytes(T, H, F, E, k))
    if need == 0:
        _check(MOE_ERR_UNSUPPORTED, "moe_mxfp8_workspace_bytes")
    ws = _ws(need, dev) if ws is None else ws
    st = lib.moe_forward_mxfp8(_ptr(x), _ptr(Wr), _ptr(bias), _ptr(W1q), _ptr(W1_scale), _ptr(W2q), _ptr(W2_scale), T,
                               H, F, E, k, float(drop_thresh), _ptr(y), _dt(y), _ptr(topk_ids), _ptr(topk_w),
                               _ptr(expert_offsets), _ptr(inv), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_forward_mxfp8")
    return y


def moe_grouped_ffn_mxfp8(x, row_token, expert_offsets, W1q, W1_scale, W2q, W2_scale, F: int, k: int, h_codes=None,
                          h_scale=None, y_perm=None, ws=None, stream=None):
    """Both expert products on MX operands from bf16 x and moe_permute's maps (the dispatched rows are quantised
    as they are copied). Returns (h_codes [F/64, T*k, 64] uint8 (k-blocked), h_scale [F/128, T*k, 4] uint8,
    y_perm [T*k, H] fp32)."""
    _arg(x, "x", (None, None), torch.bfloat16)
    T, H = x.shape
    dev = x.device
    _arg(expert_offsets, "expert_offsets", (None,), torch.int32, dev)
    E = expert_offsets.shape[0] - 1
    _arg(row_token, "row_token", (T * k,), torch.int32, dev)
    _mx_weights(W1q, W1_scale, W2q, W2_scale, E, H, F, dev)
    lib = load_library()
    h_codes = torch.empty((F // 64, T * k, 64), dtype=torch.uint8, device=dev) if h_codes is None else h_codes
    h_scale = torch.empty((F // 128, T * k, 4), dtype=torch.uint8, device=dev) if h_scale is None else h_scale
    y_perm = torch.empty((T * k, H), dtype=torch.float32, device=dev) if y_perm is None else y_perm
    _arg(h_codes, "h_codes", (F // 64, T * k, 64), torch.uint8, dev)
    _arg(h_scale, "h_scale", (F // 128, T * k, 4), torch.uint8, dev)
    _arg(y_perm, "y_perm", (T * k, H), torch.float32, dev)
    _ws_arg(ws, dev)
    ws = _ws(lib.moe_grouped_ffn_mxfp8_workspace_bytes(T, H, k), dev) if ws is None else ws
    st = lib.moe_grouped_ffn_mxfp8(_ptr(x), _ptr(row_token), _ptr(expert_offsets), _ptr(W1q), _ptr(W1_scale),
                                   _ptr(W2q), _ptr(W2_scale), T, H, F, E, k, _ptr(h_codes), _ptr(h_scale),
                                   _ptr(y_perm), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "moe_grouped_ffn_mxfp8")
    return h_codes, h_scale, y_perm


def moe_calibrate_mfma_bf16(workgroups: int, waves: int, iters: int, sink=None, stream=None,
                            random_operands: bool = False) -> int:
    """Bare bf16 MFMA loop (measurement aid), on one fixed operand pair or on pseudo-random operands per MFMA.
    Returns the FLOP count of the launch."""
    sink = torch.empty(workgroups * waves * 64, dtype=torch.float32, device="cuda") if sink is None else sink
    _arg(sink, "sink", (workgroups * waves * 64,), torch.float32)
    _check(load_library().moe_calibrate_mfma_bf16(workgroups, waves, iters, int(bool(random_operands)), _ptr(sink),
                                                  _stream(stream)),
           "moe_calibrate_mfma_bf16")
    return workgroups * waves * iters * 8 * 32768


def moe_calibrate_stream_read(buf, workgroups: int, sink=None, stream=None) -> int:
    """Streaming read of every byte of buf (measurement aid). Returns the byte count."""
    nbytes = buf.numel() * buf.element_size()
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device=buf.device) if sink is None else sink
    _arg(sink, "sink", (workgroups * 256,), torch.float32, buf.device)
    _check(load_library().moe_calibrate_stream_read(_ptr(buf), nbytes, workgroups, _ptr(sink), _stream(stream)),
           "moe_calibrate_stream_read")
    return nbytes


def moe_calibrate_gemm_kstep(mode: int, workgroups: int, steps: int, src=None, sink=None, stream=None) -> int:
    """The grouped FFN's 256x256 k-step repeated (measurement aid): mode 0 without global memory, 1 with its
    32 KB-per-step direct-to-LDS feed from src (offsets modulo src's size), 2 the feed alone.
    Returns the FLOP count of the launch (modes 0 and 1) or the bytes fed (mode 2)."""
    sink = torch.empty(workgroups * 512, dtype=torch.float32, device="cuda") if sink is None else sink
    _arg(sink, "sink", (workgroups * 512,), torch.float32)
    span = src.numel() * src.element_size() if src is not None else 0
    _check(load_library().moe_calibrate_gemm_kstep(_ptr(src), span, workgroups, steps, mode, _ptr(sink),
                                                   _stream(stream)), "moe_calibrate_gemm_kstep")
    return workgroups * steps * 32768 if mode == 2 else workgroups * steps * 4194304
