"""GPU parity of the fp8 expert weights (moe_quantize_fp8, moe_grouped_ffn_fp8,
moe_forward_fp8) against the oracle's quantisation and its layer evaluated
with the dequantised weights.

Bar: codes and scales bit-exact (codes unpacked from the tiled layout the
header documents, padding columns zero); y_perm and y within 2e-2 * rms of
the oracle's layer on the oracle's own dequantised weights; routing arrays
bit-exact; the one-call path within 2^-10 * max|y_perm| of the step-wise path
(its y_perm is kept as block-scaled fp16).
"""
import numpy as np
import pytest

import gen
import oracle
from tests.scaled16 import scaled16_bound

torch = pytest.importorskip("torch")
moe = pytest.importorskip("top_routing_grouped_gemm_amd")

pytestmark = pytest.mark.gpu

Y_TOL = 2e-2
W_TOL = 2e-6


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def unpack_tiles(buf, E, K, N):
    """Codes [E,K,N] and padding columns from the tiled layout: tiles of 128
    columns x 64 k, [E][ceil(N/128)][K/64][128][64] bytes, the 8-byte k-chunk c
    of tile column n stored at chunk c ^ (((n >> 1) & 7) ^ ((n >> 4) & 1))."""
    NB, KB = (N + 127) // 128, K // 64
    t = np.asarray(buf, dtype=np.uint8).reshape(E, NB, KB, 128, 8, 8)
    n = np.arange(128)
    swz = ((n >> 1) & 7) ^ ((n >> 4) & 1)
    where = np.arange(8)[None, :] ^ swz[:, None]          # stored chunk of k-chunk c, per column
    t = np.take_along_axis(t, where[None, None, None, :, :, None], axis=4)
    codes = t.transpose(0, 2, 4, 5, 1, 3).reshape(E, K, NB * 128)  # k = kb*64 + c*8 + byte, n = nb*128 + col
    return codes[:, :, :N], codes[:, :, N:]


def _bits(a):
    """bf16 storage bits (uint16) -> torch bf16 tensor, fp32 arrays as they are."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


def _special_columns(W, dtype):
    """Plant structure into a [E,K,N] weight draw: an all-zero column, a column
    whose maximum is exactly 448 (scale 1, so W/scale hits e4m3 ties exactly)
    and a column whose largest magnitude is negative."""
    W = W.copy()
    K = W.shape[1]
    ties = np.array([1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, -3 * 2.0 ** -10, 0.0, 448.0,
                     17.0, 18.0, 36.0, 0.3125])  # each a midpoint or exact point of the e4m3 grid
    col = np.resize(ties, K)
    col[0] = 448.0
    neg = np.asarray(gen.to_f64(W[0, :, 2], dtype), dtype=np.float64).copy()
    neg[K // 2] = -8.0 * np.abs(neg).max() - 1.0
    if dtype == "bf16":
        W[:, :, 0] = 0
        W[0, :, 1] = gen.f32_to_bf16_bits(col.astype(np.float32))
        W[0, :, 2] = gen.f32_to_bf16_bits(neg.astype(np.float32))
    else:
        W[:, :, 0] = 0.0
        W[0, :, 1] = col
        W[0, :, 2] = neg
    return W


@pytest.mark.parametrize("E,K,N,dtype,seed", [
    (3, 128, 200, "bf16", 61),    # N past a tile boundary: padded columns
    (2, 192, 136, "f32", 62),
    (1, 64, 128, "bf16", 63),     # one tile
    (5, 256, 384, "f32", 64),
])
def test_quantize_bit_exact(dev, E, K, N, dtype, seed):
    _say(f"quantize E={E} K={K} N={N} {dtype}")
    W = gen.normal(seed, 1, E * K * N, 1.0 / np.sqrt(K), dtype).reshape(E, K, N)
    W = _special_columns(W, dtype)
    Wq, sc = moe.moe_quantize_fp8(_bits(W).to(dev))
    torch.cuda.synchronize()
    codes, pad = unpack_tiles(Wq.cpu().numpy(), E, K, N)
    ref_codes, ref_sc = oracle.quantize_fp8(gen.to_f64(W, dtype))
    assert np.array_equal(sc.cpu().numpy(), ref_sc)
    assert np.array_equal(codes, ref_codes)
    assert not pad.any()
    # the planted tie column quantises with scale 1: the even code of each tie
    assert ref_sc[0, 1] == 1.0


@pytest.mark.parametrize("name,which", [("decode", "W1"), ("decode", "W2")])
def test_quantize_full_size_sampled_experts(dev, name, which):
    """The full expert stacks of the decode workload are quantised on the GPU;
    the oracle re-quantises a sample of experts independently."""
    I = gen.make_inputs(name)
    d = gen.to_device(I, dev)
    W = d[which]
    E, K, N = W.shape
    _say(f"quantize {name} {which}: E={E} K={K} N={N}")
    Wq, sc = moe.moe_quantize_fp8(W)
    torch.cuda.synchronize()
    buf = Wq.cpu().numpy().reshape(E, -1)
    for e in (0, E // 2 + 1, E - 1):
        codes, pad = unpack_tiles(buf[e], 1, K, N)
        getter = I.W1 if which == "W1" else I.W2
        rc, rs = oracle.quantize_fp8(I.f64(getter(e, e + 1)))
        assert np.array_equal(sc[e].cpu().numpy(), rs[0]), e
        assert np.array_equal(codes, rc), e
        assert not pad.any()


def _deq_getter(getter, f64, keep=True):
    """Expert e's dequantised fp8 weights (the oracle's quantiser); keep=False: no cache (each expert once)."""
    cache = {}

    def W(e):
        if e in cache:
            return cache[e]
        c, s = oracle.quantize_fp8(f64(getter(e, e + 1)))
        v = oracle.dequantize_fp8(c, s)[0]
        if keep:
            cache[e] = v
        return v
    return W


def _check_y(y_gpu, y_ref, tol=Y_TOL):
    rms = float(np.sqrt((y_ref ** 2).mean()))
    err = float(np.abs(y_gpu - y_ref).max())
    assert err <= tol * rms, f"max-abs error {err:.3e} > {tol} * rms {rms:.3e}"
    return err / rms


SMALL = [
    dict(T=300, H=128, F=192, E=6, k=2, zipf=1.2, seed=71),      # ~100 rows per expert: the large shape
    dict(T=200, H=256, F=320, E=8, k=2, zipf=1.2, seed=72),      # ~50 rows: both shapes by group size
    dict(T=64, H=128, F=256, E=16, k=2, seed=73),                # ~8 rows: the streaming shape
    dict(T=50, H=384, F=128, E=4, k=3, drop=0.1, seed=74),       # drop threshold, mixed sizes
    dict(T=1, H=128, F=128, E=8, k=2, seed=75),                  # one token
]


@pytest.mark.parametrize("over", SMALL, ids=[f"small-{i}" for i in range(len(SMALL))])
def test_fp8_layer_small(dev, over):
    I = gen.make_inputs("tiny", dtype="bf16", **over)
    _say(f"fp8 layer {over}")
    d = gen.to_device(I, dev)
    W1q, s1 = moe.moe_quantize_fp8(d["W1"])
    W2q, s2 = moe.moe_quantize_fp8(d["W2"])
    ids, w = moe.moe_route(d["x"], d["Wr"], d["bias"], I.k, I.drop)
    x_perm, off, row_token, inv = moe.moe_permute(d["x"], ids, w, I.E)
    y_perm = moe.moe_grouped_ffn_fp8(x_perm, off, W1q, s1, W2q, s2, I.T, I.k)
    y_steps = moe.moe_combine(y_perm, inv, w)
    ids2 = torch.empty_like(ids)
    inv2 = torch.empty_like(inv)
    y = moe.moe_forward_fp8(d["x"], d["Wr"], d["bias"], W1q, s1, W2q, s2, I.k, I.drop, topk_ids=ids2, inv=inv2)
    torch.cuda.synchronize()

    W1 = _deq_getter(I.W1, I.f64)
    W2 = _deq_getter(I.W2, I.f64)
    ref = oracle.forward(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), W1, W2, I.k, I.drop)
    assert np.array_equal(ids.cpu().numpy(), ref.route.ids)
    assert np.array_equal(off.cpu().numpy(), ref.dispatch.offsets)
    assert torch.equal(ids, ids2) and torch.equal(inv, inv2)
    A = int(ref.dispatch.offsets[-1])
    _check_y(y_perm[:A].double().cpu().numpy(), ref.y_perm)
    _check_y(y_steps.double().cpu().numpy(), ref.y)
    _check_y(y.double().cpu().numpy(), ref.y)
    bound = 2.0 ** -10 * float(y_perm[:A].abs().max()) if A else 0.0  # block-scaled fp16 y_perm
    assert float((y - y_steps).abs().max()) <= bound
    if I.H % 32 == 0:  # and element by element
        eb = scaled16_bound(y_perm, A, inv, w, y_steps)
        assert bool(((y - y_steps).abs().double() <= eb).all()), "one-call y outside the fp16 rounding bound"


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_fp8_full_workload(dev, name):
    """Full-size layer on fp8 experts, every token: routing arrays bit-exact, y against the oracle's layer on
    the dequantised experts (built one expert at a time)."""
    I = gen.make_inputs(name)
    _say(f"fp8 full {name}: T={I.T} H={I.H} F={I.F} E={I.E} k={I.k}")
    d = gen.to_device(I, dev)
    W1q, s1 = moe.moe_quantize_fp8(d["W1"])
    W2q, s2 = moe.moe_quantize_fp8(d["W2"])
    ids = torch.empty((I.T, I.k), dtype=torch.int32, device=dev)
    w = torch.empty((I.T, I.k), dtype=torch.float32, device=dev)
    y = moe.moe_forward_fp8(d["x"], d["Wr"], d["bias"], W1q, s1, W2q, s2, I.k, I.drop, topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    r = oracle.route(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), I.k, I.drop)
    assert np.array_equal(ids.cpu().numpy(), r.ids)
    assert np.abs(w.cpu().numpy() - r.w).max() <= W_TOL
    y_n = y.double().cpu().numpy()
    del y, d, W1q, W2q
    torch.cuda.empty_cache()
    ref = oracle.forward(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), _deq_getter(I.W1, I.f64, keep=False),
                         _deq_getter(I.W2, I.f64, keep=False), I.k, I.drop)
    rel = _check_y(y_n, ref.y)
    _say(f"{name} fp8: y max-abs/rms {rel:.3e} on all {I.T} tokens")
