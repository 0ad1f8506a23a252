"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before launching anything (no GPU needed:
every call here returns at argument validation)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

moe = pytest.importorskip("top_routing_grouped_gemm_amd")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return moe.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_forward",
                          "moe_workspace_bytes", "moe_strerror"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe.h but not exported"
    assert set(moe.EXPORTS) == set(names)


def test_strerror_and_version(lib):
    for st in (0, -1, -2, -3, -4):
        assert moe.strerror(st).startswith("MOE_")
    assert "unknown" in moe.strerror(7)
    assert re.match(r"^\d+\.\d+\.\d+$", moe.version())


def test_workspace_queries(lib):
    bf16, f32 = 1, 0
    T, H, F, E, k = 8192, 2048, 768, 128, 8
    n = lib.moe_workspace_bytes(T, H, F, E, k, 0, bf16)
    # at least x_perm (bf16) + y_perm (fp32) + h (bf16)
    assert n >= T * k * (H * 2 + H * 4 + F * 2)
    assert lib.moe_workspace_bytes(T, H, F, E, k, 4096, bf16) > n  # shared expert adds h_sh, y_sh
    assert lib.moe_workspace_bytes(T, H, F, E, k, 0, f32) > n
    assert lib.moe_permute_workspace_bytes(T, E, k) == ((T * k + 1023) // 1024) * E * 4  # per-chunk counts, 1024 slots a chunk
    assert lib.moe_ffn_workspace_bytes(T, F, E, k, 0, bf16) >= T * k * F * 2
    for bad in [(0, H, F, E, k), (T, 0, F, E, k), (T, H, 0, E, k), (T, H, F, 0, k), (T, H, F, E, 0),
                (T, H, F, E, E + 1), (T, 12, F, E, k), (T, H, F, 2048, k), (T, H, F, 64, 40)]:
        assert lib.moe_workspace_bytes(*bad, 0, bf16) == 0, bad
    assert lib.moe_workspace_bytes(T, H, F, E, k, 0, 7) == 0
    assert lib.moe_workspace_bytes(T, H, F, E, k, 12, bf16) == 0


def _p(v=0x1000):
    return ctypes.c_void_p(v)  # never dereferenced: validation fails first


def test_route_rejects(lib):
    N = None
    ok = dict(x=_p(), Wr=_p(), b=N, T=4, H=8, E=4, k=2, drop=0.0, dt=1, ids=_p(), w=_p(), ws=N, wsb=0, s=N)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.moe_route(a["x"], a["Wr"], a["b"], a["T"], a["H"], a["E"], a["k"], a["drop"], a["dt"], a["ids"],
                             a["w"], a["ws"], a["wsb"], a["s"])

    assert call(T=0) == moe.MOE_ERR_INVALID_ARG
    assert call(k=5) == moe.MOE_ERR_INVALID_ARG
    assert call(k=0) == moe.MOE_ERR_INVALID_ARG
    assert call(x=N) == moe.MOE_ERR_INVALID_ARG
    assert call(ids=N) == moe.MOE_ERR_INVALID_ARG
    assert call(drop=0.6) == moe.MOE_ERR_INVALID_ARG   # > 1/k
    assert call(drop=-0.1) == moe.MOE_ERR_INVALID_ARG
    assert call(drop=float("nan")) == moe.MOE_ERR_INVALID_ARG
    assert call(dt=3) == moe.MOE_ERR_INVALID_ARG
    assert call(H=12) == moe.MOE_ERR_UNSUPPORTED
    assert call(E=2000, k=2) == moe.MOE_ERR_UNSUPPORTED
    assert call(E=1025, k=2) == moe.MOE_ERR_UNSUPPORTED   # one past the expert limit
    assert call(T=4, E=64, k=33) == moe.MOE_ERR_UNSUPPORTED  # one past the top-k limit
    # a split router (few tokens, long H) needs its partial-logit workspace
    need = lib.moe_route_workspace_bytes(32, 2048, 128, 1)
    assert need == 32 * 32 * 128 * 4
    assert call(T=32, H=2048, E=128, k=8) == moe.MOE_ERR_WORKSPACE
    assert call(T=32, H=2048, E=128, k=8, ws=_p(), wsb=need - 1) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_route_workspace_bytes(8192, 2048, 128, 1) == 2 * 8192 * 128 * 4   # 256 token blocks x 2 splits
    assert lib.moe_route_workspace_bytes(65536, 2048, 128, 1) == 0   # enough token blocks: no split
    assert lib.moe_route_workspace_bytes(32, 2048, 128, 0) == 0     # fp32 router never splits


def test_capacity_rejects(lib):
    N = None
    bf16 = 1
    # workspace queries: router shapes only (bf16, E % 8 == 0, E <= 256, H % 64 == 0)
    assert lib.moe_route_capacity_workspace_bytes(8192, 2048, 128, bf16) > 8192 * 128 * 4
    assert lib.moe_route_capacity_workspace_bytes(64, 64, 4, 0) == 0          # fp32: unsupported
    assert lib.moe_route_capacity_workspace_bytes(64, 96, 8, bf16) == 0       # H % 64 != 0
    assert lib.moe_select_capacity_workspace_bytes(100, 16) > 0
    assert lib.moe_select_capacity_workspace_bytes(100, 2000) == 0

    def route(**kw):
        a = dict(x=_p(), Wr=_p(), b=N, T=2048, H=5120, E=64, k=2, drop=0.0, f=1.2, dt=bf16, ids=_p(), w=_p(),
                 ws=N, wsb=0, s=N)
        a.update(kw)
        return lib.moe_route_capacity(a["x"], a["Wr"], a["b"], a["T"], a["H"], a["E"], a["k"], a["drop"], a["f"],
                                      a["dt"], a["ids"], a["w"], a["ws"], a["wsb"], a["s"])

    assert route(f=0.0) == moe.MOE_ERR_INVALID_ARG
    assert route(f=float("nan")) == moe.MOE_ERR_INVALID_ARG
    assert route(f=float("inf")) == moe.MOE_ERR_INVALID_ARG
    assert route(f=0.5) == moe.MOE_ERR_UNSUPPORTED        # cap 32: 64 experts could all fill, none left
    assert route(T=64, H=64, E=4, k=2) == moe.MOE_ERR_UNSUPPORTED   # cap 39: only one expert is sure to have room
    assert route(dt=0, T=64, H=64, E=64, k=2) == moe.MOE_ERR_UNSUPPORTED   # fp32 router: no logits path
    assert route() == moe.MOE_ERR_WORKSPACE
    assert route(ids=N) == moe.MOE_ERR_INVALID_ARG

    def select(**kw):
        a = dict(lg=_p(), T=100, E=16, k=2, drop=0.0, cap=20, ids=_p(), w=_p(), ws=_p(), wsb=1 << 20, s=N)
        a.update(kw)
        return lib.moe_select_capacity(a["lg"], a["T"], a["E"], a["k"], a["drop"], a["cap"], a["ids"], a["w"],
                                       a["ws"], a["wsb"], a["s"])

    assert select(cap=0) == moe.MOE_ERR_INVALID_ARG
    assert select(cap=13) == moe.MOE_ERR_UNSUPPORTED      # 16 - 200 // 13 = 1 < 2
    assert select(wsb=1) == moe.MOE_ERR_WORKSPACE
    assert select(lg=N) == moe.MOE_ERR_INVALID_ARG
    assert select(drop=0.7) == moe.MOE_ERR_INVALID_ARG


def test_permute_ffn_combine_forward_reject(lib):
    N = None
    # permute: undersized workspace
    need = lib.moe_permute_workspace_bytes(64, 4, 2)
    assert lib.moe_permute(_p(), _p(), _p(), 64, 8, 4, 2, 1, _p(), _p(), _p(), _p(), _p(), need - 1, N) \
        == moe.MOE_ERR_WORKSPACE
    assert lib.moe_permute(_p(), _p(), _p(), 64, 8, 4, 2, 1, _p(), N, _p(), _p(), _p(), need, N) \
        == moe.MOE_ERR_INVALID_ARG
    # grouped ffn: shared expert needs all of x, W2s, y_shared; Fs multiple of 8
    need = lib.moe_ffn_workspace_bytes(64, 16, 4, 2, 0, 1)
    assert lib.moe_grouped_ffn(_p(), _p(), _p(), _p(), 64, 8, 16, 4, 2, 1, _p(), N, _p(), N, 8, N, _p(), need, N) \
        == moe.MOE_ERR_INVALID_ARG
    need_s = lib.moe_ffn_workspace_bytes(64, 16, 4, 2, 8, 1)
    assert lib.moe_grouped_ffn(_p(), _p(), _p(), _p(), 64, 8, 16, 4, 2, 1, _p(), _p(), _p(), _p(), 12, _p(), _p(),
                               need_s, N) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_grouped_ffn(_p(), _p(), _p(), _p(), 64, 8, 16, 4, 2, 1, _p(), _p(), _p(), _p(), 8, _p(), _p(),
                               need, N) == moe.MOE_ERR_WORKSPACE
    # combine
    assert lib.moe_combine(_p(), _p(), _p(), N, 0, 8, 2, 0, _p(), N) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(_p(), _p(), _p(), N, 4, 6, 2, 0, _p(), N) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_combine(_p(), N, _p(), N, 4, 8, 2, 0, _p(), N) == moe.MOE_ERR_INVALID_ARG
    # forward
    need = lib.moe_workspace_bytes(64, 8, 16, 4, 2, 0, 1)
    args = [_p(), _p(), N, _p(), _p(), N, N, 0, 64, 8, 16, 4, 2, 0.0, 1, _p(), 0, N, N, N, N, _p(), need, N]
    bad = list(args)
    bad[22] = need - 1
    assert lib.moe_forward(*bad) == moe.MOE_ERR_WORKSPACE
    bad = list(args)
    bad[5] = _p()  # W1s without W2s
    assert lib.moe_forward(*bad) == moe.MOE_ERR_INVALID_ARG
    bad = list(args)
    bad[13] = 0.7
    assert lib.moe_forward(*bad) == moe.MOE_ERR_INVALID_ARG
    bad = list(args)
    bad[16] = 5
    assert lib.moe_forward(*bad) == moe.MOE_ERR_INVALID_ARG


def test_fp8_rejects(lib):
    N = None
    bf16 = 1
    # tiled code bytes: E * ceil(N/128)*128 * K; K must be a multiple of 64
    assert lib.moe_fp8_weight_bytes(128, 2048, 768) == 128 * 768 * 2048
    assert lib.moe_fp8_weight_bytes(2, 64, 100) == 2 * 128 * 64
    assert lib.moe_fp8_weight_bytes(2, 96, 128) == 0
    assert lib.moe_fp8_weight_bytes(0, 64, 128) == 0
    assert lib.moe_quantize_fp8(_p(), 2, 96, 128, bf16, _p(), _p(), N) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_quantize_fp8(_p(), 2, 64, 128, 5, _p(), _p(), N) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_fp8(_p(), 0, 64, 128, bf16, _p(), _p(), N) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_fp8(_p(), 2, 64, 128, bf16, N, _p(), N) == moe.MOE_ERR_INVALID_ARG
    # grouped ffn: H, F multiples of 64 and >= 128
    need = lib.moe_ffn_workspace_bytes(64, 256, 4, 2, 0, bf16)

    def ffn(H=256, F=256, ws=need, y=_p()):
        return lib.moe_grouped_ffn_fp8(_p(), _p(), _p(), _p(), _p(), _p(), 64, H, F, 4, 2, y, _p(), ws, N)

    assert ffn(H=96) == moe.MOE_ERR_UNSUPPORTED
    assert ffn(F=64) == moe.MOE_ERR_UNSUPPORTED
    assert ffn(ws=need - 1) == moe.MOE_ERR_WORKSPACE
    assert ffn(y=N) == moe.MOE_ERR_INVALID_ARG
    # forward
    need = lib.moe_workspace_bytes(64, 256, 256, 4, 2, 0, bf16)
    args = [_p(), _p(), N, _p(), _p(), _p(), _p(), 64, 256, 256, 4, 2, 0.0, _p(), 0, N, N, N, N, _p(), need, N]
    assert len(args) == len(lib.moe_forward_fp8.argtypes)
    bad = list(args)
    bad[20] = need - 1
    assert lib.moe_forward_fp8(*bad) == moe.MOE_ERR_WORKSPACE
    bad = list(args)
    bad[4] = N  # W1 scales
    assert lib.moe_forward_fp8(*bad) == moe.MOE_ERR_INVALID_ARG
    bad = list(args)
    bad[8] = 200  # H % 64 != 0
    assert lib.moe_forward_fp8(*bad) == moe.MOE_ERR_UNSUPPORTED
    bad = list(args)
    bad[12] = 0.7
    assert lib.moe_forward_fp8(*bad) == moe.MOE_ERR_INVALID_ARG


def test_mxfp8_rejects(lib):
    N = None
    bf16 = 1
    assert lib.moe_mxfp8_weight_bytes(128, 2048, 768) == 128 * 768 * 2048
    assert lib.moe_mxfp8_scale_bytes(128, 2048, 768) == 128 * 16 * 768 * 4
    assert lib.moe_mxfp8_weight_bytes(2, 64, 128) == 0                    # K % 128 != 0
    assert lib.moe_mxfp8_scale_bytes(2, 128, 100) == 2 * 1 * 128 * 4      # N padded to 128
    assert lib.moe_quantize_mxfp8(_p(), 2, 64, 128, bf16, _p(), _p(), N) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_quantize_mxfp8(_p(), 2, 128, 128, 9, _p(), _p(), N) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_mxfp8(_p(), 2, 128, 128, bf16, _p(), N, N) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_mxfp8_rows(_p(), 4, 96, bf16, _p(), _p(), N) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_quantize_mxfp8_rows(_p(), 0, 128, bf16, _p(), _p(), N) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_mxfp8_workspace_bytes(64, 256, 256, 4, 2) > 0
    assert lib.moe_mxfp8_workspace_bytes(64, 192, 256, 4, 2) == 0          # H % 128 != 0
    assert lib.moe_mxfp8_workspace_bytes(64, 256, 192, 4, 2) == 0          # F % 128 != 0
    assert lib.moe_grouped_ffn_mxfp8_workspace_bytes(64, 256, 2) == 64 * 256 + 2 * 64 * 4
    assert lib.moe_grouped_ffn_mxfp8_workspace_bytes(64, 192, 2) == 0
    need = lib.moe_mxfp8_workspace_bytes(64, 256, 256, 4, 2)
    args = [_p(), _p(), N, _p(), _p(), _p(), _p(), 64, 256, 256, 4, 2, 0.0, _p(), 0, N, N, N, N, _p(), need, N]
    assert len(args) == len(lib.moe_forward_mxfp8.argtypes)
    bad = list(args)
    bad[20] = need - 1
    assert lib.moe_forward_mxfp8(*bad) == moe.MOE_ERR_WORKSPACE
    bad = list(args)
    bad[6] = N
    assert lib.moe_forward_mxfp8(*bad) == moe.MOE_ERR_INVALID_ARG
    bad = list(args)
    bad[8] = 320
    assert lib.moe_forward_mxfp8(*bad) == moe.MOE_ERR_UNSUPPORTED
    bad = list(args)
    bad[14] = 4
    assert lib.moe_forward_mxfp8(*bad) == moe.MOE_ERR_INVALID_ARG


def test_binding_raises_without_library(tmp_path):
    with pytest.raises(ImportError):
        moe.load_library(str(tmp_path / "missing.so"))


# ------------------------------------------------ binding argument checks --
def test_binding_rejects_mismatched_tensors(lib):
    """The Python binding validates every tensor's dtype, shape and device against the sizes of the call before a
    pointer reaches the library (a short or mistyped buffer would make a kernel read or write out of bounds).
    CPU tensors get through these checks only when everything else is right; the last check refuses them."""
    torch = pytest.importorskip("torch")
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    T, H, F, E, k = 8, 64, 32, 4, 2
    x = torch.zeros((T, H), dtype=bf)
    Wr = torch.zeros((H, E), dtype=bf)
    W1 = torch.zeros((E, H, F), dtype=bf)
    W2 = torch.zeros((E, F, H), dtype=bf)
    ids = torch.zeros((T, k), dtype=i32)
    w = torch.zeros((T, k), dtype=f32)

    def raises(exc, match, fn, *a, **kw):
        with pytest.raises(exc, match=match):
            fn(*a, **kw)

    # moe_forward: operand dtypes and shapes
    raises(TypeError, "W1 has dtype", moe.moe_forward, x, Wr, None, W1.float(), W2, k)
    raises(TypeError, "x has dtype", moe.moe_forward, x.half(), Wr, None, W1, W2, k)
    raises(ValueError, "Wr has shape", moe.moe_forward, x, Wr[:32], None, W1, W2, k)
    raises(ValueError, "W2 has shape", moe.moe_forward, x, Wr, None, W1, W2.transpose(1, 2).contiguous(), k)
    raises(ValueError, "W1 has shape", moe.moe_forward, x, Wr, None, W1[:3], W2, k)
    raises(ValueError, "bias has shape", moe.moe_forward, x, Wr, torch.zeros(E + 1), W1, W2, k)
    raises(TypeError, "bias has dtype", moe.moe_forward, x, Wr, torch.zeros(E, dtype=torch.float64), W1, W2, k)
    raises(ValueError, "y has shape", moe.moe_forward, x, Wr, None, W1, W2, k, y=torch.zeros((T - 1, H)))
    raises(ValueError, "topk_ids has shape", moe.moe_forward, x, Wr, None, W1, W2, k, topk_ids=ids[:, :1].clone())
    raises(TypeError, "inv has dtype", moe.moe_forward, x, Wr, None, W1, W2, k, inv=ids.long())
    raises(ValueError, "expert_offsets has shape", moe.moe_forward, x, Wr, None, W1, W2, k,
           expert_offsets=torch.zeros(E, dtype=i32))
    raises(ValueError, "W2s has shape", moe.moe_forward, x, Wr, None, W1, W2, k, W1s=torch.zeros((H, 16), dtype=bf),
           W2s=torch.zeros((8, H), dtype=bf))
    raises(ValueError, "both W1s and W2s", moe.moe_forward, x, Wr, None, W1, W2, k,
           W1s=torch.zeros((H, 16), dtype=bf))
    raises(TypeError, "ws has dtype", moe.moe_forward, x, Wr, None, W1, W2, k, ws=torch.zeros(16, dtype=f32))
    raises(ValueError, "must be on the GPU", moe.moe_forward, x, Wr, None, W1, W2, k)  # everything else is right

    # moe_route / moe_permute / moe_grouped_ffn / moe_combine
    raises(ValueError, "Wr has shape", moe.moe_route, x, torch.zeros((H + 8, E), dtype=bf), None, k)
    raises(ValueError, "topk_w has shape", moe.moe_route, x, Wr, None, k, topk_w=torch.zeros((T, k + 1)))
    raises(ValueError, "must be on the GPU", moe.moe_route, x, Wr, None, k)
    raises(ValueError, "x_perm has shape", moe.moe_permute, x, ids, w, E, x_perm=torch.zeros((T * k - 1, H), dtype=bf))
    raises(TypeError, "x_perm has dtype", moe.moe_permute, x, ids, w, E, x_perm=torch.zeros((T * k, H)))
    raises(ValueError, "row_token has shape", moe.moe_permute, x, ids, w, E, row_token=torch.zeros(T, dtype=i32))
    raises(TypeError, "topk_ids has dtype", moe.moe_permute, x, ids.long(), w, E)
    x_perm = torch.zeros((T * k, H), dtype=bf)
    off = torch.zeros(E + 1, dtype=i32)
    raises(ValueError, "x_perm has shape", moe.moe_grouped_ffn, x_perm[:-1].contiguous(), off, W1, W2, T, k)
    raises(ValueError, "expert_offsets has shape", moe.moe_grouped_ffn, x_perm, off[:-1].contiguous(), W1, W2, T, k)
    raises(TypeError, "W2 has dtype", moe.moe_grouped_ffn, x_perm, off, W1, W2.float(), T, k)
    raises(ValueError, "y_perm has shape", moe.moe_grouped_ffn, x_perm, off, W1, W2, T, k,
           y_perm=torch.zeros((T * k, H - 8)))
    raises(TypeError, "y_perm has dtype", moe.moe_grouped_ffn, x_perm, off, W1, W2, T, k,
           y_perm=torch.zeros((T * k, H), dtype=bf))
    raises(ValueError, "must be on the GPU", moe.moe_grouped_ffn, x_perm, off, W1, W2, T, k)
    y_perm = torch.zeros((T * k, H))
    raises(ValueError, "topk_w has shape", moe.moe_combine, y_perm, ids, w[:, :1].contiguous())
    raises(ValueError, "y_shared has shape", moe.moe_combine, y_perm, ids, w, y_shared=torch.zeros((T, H + 8)))
    raises(TypeError, "y has dtype", moe.moe_combine, y_perm, ids, w, y=torch.zeros((T, H), dtype=torch.float16))
    raises(ValueError, "must be on the GPU", moe.moe_combine, y_perm, ids, w)

    # quantised expert formats: codes and scales must have the sizes the quantisers write
    W1q = torch.zeros(moe.moe_fp8_weight_bytes(E, H, F), dtype=torch.uint8)
    W2q = torch.zeros(moe.moe_fp8_weight_bytes(E, F, H), dtype=torch.uint8)
    s1, s2 = torch.zeros((E, F)), torch.zeros((E, H))
    raises(ValueError, "W1q has shape", moe.moe_forward_fp8, x, Wr, None, W1q[:-1].contiguous(), s1, W2q, s2, k)
    raises(ValueError, "W2_scale has shape", moe.moe_forward_fp8, x, Wr, None, W1q, s1, W2q, s2[:, :-1].contiguous(),
           k)
    raises(ValueError, "must be on the GPU", moe.moe_forward_fp8, x, Wr, None, W1q, s1, W2q, s2, k)
    raises(ValueError, "Wq has shape", moe.moe_quantize_fp8, W1, Wq=W1q[:-1].contiguous())


def test_noalloc_limits(lib):
    """moe_forward_noalloc checks its arguments like moe_forward and refuses, before touching the GPU, a batch
    whose buffers exceed its 64 MiB scratch array."""
    N = None
    bf16 = 1

    def call(T, H, F, E, k, x=_p(), y=_p(), Fs=0, W1s=N, W2s=N, drop=0.0):
        return lib.moe_forward_noalloc(x, _p(), N, _p(), _p(), W1s, W2s, Fs, T, H, F, E, k, drop, bf16, y, bf16,
                                       N, N, N, N, N)

    assert call(8192, 2048, 768, 128, 8) == moe.MOE_ERR_UNSUPPORTED      # prefill: ~370 MB of buffers
    assert call(2048, 2048, 768, 128, 8) == moe.MOE_ERR_UNSUPPORTED      # 16,384 assignments
    assert call(0, 2048, 768, 128, 8) == moe.MOE_ERR_INVALID_ARG
    assert call(32, 2048, 768, 128, 8, x=N) == moe.MOE_ERR_INVALID_ARG
    assert call(32, 2048, 768, 128, 8, y=N) == moe.MOE_ERR_INVALID_ARG
    assert call(32, 2048, 768, 128, 8, drop=0.5) == moe.MOE_ERR_INVALID_ARG
    assert call(32, 2048, 768, 128, 8, Fs=64, W1s=_p()) == moe.MOE_ERR_INVALID_ARG   # W2s missing
    assert call(32, 12, 768, 128, 8) == moe.MOE_ERR_UNSUPPORTED


def test_grouped_ffn_fused_limits(lib):
    """The on-chip-h grouped FFN refuses, before any launch, the shapes whose h does not fit (F > 768, F % 256 != 0,
    H % 256 != 0) and non-bf16 operands."""
    N = None

    def call(T=64, H=256, F=256, E=4, k=2, dt=1, x=_p(), y=_p()):
        return lib.moe_grouped_ffn_fused(x, _p(), _p(), _p(), T, H, F, E, k, dt, y, N)

    assert call(F=1024) == moe.MOE_ERR_UNSUPPORTED
    assert call(F=320) == moe.MOE_ERR_UNSUPPORTED
    assert call(H=384) == moe.MOE_ERR_UNSUPPORTED
    assert call(dt=0) == moe.MOE_ERR_UNSUPPORTED
    assert call(x=N) == moe.MOE_ERR_INVALID_ARG
    assert call(y=N) == moe.MOE_ERR_INVALID_ARG
    assert call(T=0) == moe.MOE_ERR_INVALID_ARG


def test_calibrate_mfma_rejects(lib):
    """The MFMA calibration aid refuses bad sizes and operand modes before any launch."""
    N = None
    assert lib.moe_calibrate_mfma_bf16(256, 8, 16, 2, _p(), N) == moe.MOE_ERR_INVALID_ARG    # operands 0 or 1
    assert lib.moe_calibrate_mfma_bf16(256, 8, 16, -1, _p(), N) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calibrate_mfma_bf16(256, 9, 16, 0, _p(), N) == moe.MOE_ERR_INVALID_ARG    # 1..8 waves
    assert lib.moe_calibrate_mfma_bf16(0, 8, 16, 1, _p(), N) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calibrate_mfma_bf16(256, 8, 0, 1, _p(), N) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calibrate_mfma_bf16(256, 8, 16, 1, N, N) == moe.MOE_ERR_INVALID_ARG      # no sink


def test_calibrate_gemm_kstep_rejects(lib):
    """The k-step calibration aid refuses bad modes and feed spans before any launch."""
    N = None
    assert lib.moe_calibrate_gemm_kstep(N, 0, 256, 16, 3, _p(), N) == moe.MOE_ERR_INVALID_ARG     # no mode 3
    assert lib.moe_calibrate_gemm_kstep(N, 0, 256, 16, 1, _p(), N) == moe.MOE_ERR_INVALID_ARG     # feed needs src
    assert lib.moe_calibrate_gemm_kstep(_p(), 16384, 256, 16, 1, _p(), N) == moe.MOE_ERR_INVALID_ARG  # span < 32 KB
    assert lib.moe_calibrate_gemm_kstep(_p(), 40008, 256, 16, 2, _p(), N) == moe.MOE_ERR_INVALID_ARG  # span % 16 != 0
    assert lib.moe_calibrate_gemm_kstep(N, 0, 0, 16, 0, _p(), N) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_calibrate_gemm_kstep(N, 0, 256, 16, 0, N, N) == moe.MOE_ERR_INVALID_ARG
