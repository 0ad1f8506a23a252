"""GPU parity of the MX fp8 path (moe_quantize_mxfp8, moe_quantize_mxfp8_rows,
moe_grouped_ffn_mxfp8, moe_forward_mxfp8) against the oracle's MX
quantisation and its MX layer.

Bar:
* weight and row codes and scale bytes bit-exact (unpacked by the layouts the
  header documents);
* routing ids, offsets and row order bit-exact;
* the expert's re-quantised SiLU output h: codes and scales equal to the
  oracle's, except where the oracle's fp64 h lies within the matrix cores'
  accumulation error bound of an E4M3 rounding boundary -- a decision that
  floating point takes and that neither side can take in the other's
  arithmetic (the hardware rounds inside its 64-k product blocks); there the
  GPU's code must be one that the bound interval rounds to;
* y_perm and y within 2e-2 * rms of the oracle's MX layer, widened only by
  the effect of those validated neighbouring codes through W2;
* the one-call path within 2^-10 * max|y_perm| of the step-wise path, and
  reruns bit-identical.
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


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _bits(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


def unpack_weight_codes(buf, E, K, N):
    """[E][NB][K/64][128 n][64 k] tiles, 16-byte chunk c of column n at
    c ^ (((n >> 1) & 3) ^ ((n >> 3) & 1)) -> [E][K][N] and the padding columns."""
    NB, KB = (N + 127) // 128, K // 64
    t = np.asarray(buf, dtype=np.uint8).reshape(E, NB, KB, 128, 4, 16)
    n = np.arange(128)
    where = np.arange(4)[None, :] ^ (((n >> 1) & 3) ^ ((n >> 3) & 1))[:, None]
    t = np.take_along_axis(t, where[None, None, None, :, :, None], axis=4)
    codes = t.transpose(0, 2, 4, 5, 1, 3).reshape(E, K, NB * 128)
    return codes[:, :, :N], codes[:, :, N:]


def unpack_weight_scales(buf, E, K, N):
    """byte of (e, n, block b) at ((e*(K/128) + b/4)*Npad + n)*4 + b%4 -> [E][K/32][N]."""
    NB, KB = (N + 127) // 128, K // 128
    s = np.asarray(buf, dtype=np.uint8).reshape(E, KB, NB * 128, 4)
    s = s.transpose(0, 1, 3, 2).reshape(E, KB * 4, NB * 128)
    return s[:, :, :N], s[:, :, N:]


def unpack_row_scales(buf, T, H):
    """byte of (t, block b) at ((b/4)*T + t)*4 + b%4 -> [T][H/32]."""
    s = np.asarray(buf, dtype=np.uint8).reshape(H // 128, T, 4)
    return s.transpose(1, 0, 2).reshape(T, H // 32)


@pytest.mark.parametrize("E,K,N,dtype,seed", [(2, 256, 200, "bf16", 81), (3, 128, 128, "f32", 82),
                                              (1, 384, 136, "bf16", 83)])
def test_mx_weights_bit_exact(dev, E, K, N, dtype, seed):
    _say(f"mx weights E={E} K={K} N={N} {dtype}")
    W = gen.normal(seed, 1, E * K * N, 1.0 / np.sqrt(K), dtype).reshape(E, K, N)
    # planted: an all-zero block, a block with maximum exactly 448 (scale 1: E4M3 ties land exactly), tiny values
    Wf = gen.to_f64(W, dtype).astype(np.float32)
    Wf[:, 0:32, 0] = 0.0
    Wf[:, 32:64, 1] = np.resize(np.array([448.0, 1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, 17.0, 36.0]), 32)
    Wf[:, 64:96, 2] *= 2.0 ** -20
    W = gen.f32_to_bf16_bits(Wf) if dtype == "bf16" else Wf
    Wq, Ws = moe.moe_quantize_mxfp8(_bits(W).to(dev))
    torch.cuda.synchronize()
    codes, pad = unpack_weight_codes(Wq.cpu().numpy(), E, K, N)
    scales, spad = unpack_weight_scales(Ws.cpu().numpy(), E, K, N)
    ref_c, ref_s = oracle.quantize_mx(gen.to_f64(W, dtype), axis=1)
    assert np.array_equal(scales, ref_s)
    assert np.array_equal(codes, ref_c)
    assert not pad.any() and (spad == 127).all()


@pytest.mark.parametrize("T,H,dtype,seed", [(5, 256, "bf16", 84), (64, 128, "f32", 85), (33, 2048, "bf16", 86)])
def test_mx_rows_bit_exact(dev, T, H, dtype, seed):
    _say(f"mx rows T={T} H={H} {dtype}")
    x = gen.normal(seed, 2, T * H, 1.0, dtype).reshape(T, H)
    xf = gen.to_f64(x, dtype).astype(np.float32)
    xf[0, 0:32] = 0.0
    xf[-1, 32:64] = np.resize(np.array([448.0, 1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, 17.0]), 32)
    x = gen.f32_to_bf16_bits(xf) if dtype == "bf16" else xf
    xq, xs = moe.moe_quantize_mxfp8_rows(_bits(x).to(dev))
    torch.cuda.synchronize()
    ref_c, ref_s = oracle.quantize_mx(gen.to_f64(x, dtype), axis=1)
    assert np.array_equal(unpack_row_scales(xs.cpu().numpy(), T, H), ref_s)
    assert np.array_equal(xq.cpu().numpy(), ref_c)


def _mx_getter(getter, f64):
    cache = {}

    def W(e):
        if e not in cache:
            c, s = oracle.quantize_mx(f64(getter(e, e + 1)[0]), axis=0)
            cache[e] = oracle.dequantize_mx(c, s, axis=0)
        return cache[e]
    return W


# The fp8 matrix cores round inside each 64-k product block: an in-bounds probe
# of chained v_mfma_scale_f32_32x32x64_f8f6f4 measured errors up to 5.3e-5 of
# the sum of the products' magnitudes (fp32 rounding alone would give ~6e-8).
# The bound used for h is 2^-12 of that sum (4.6x the measurement), plus the
# SiLU's own float32 evaluation (|silu'| <= 1.1; 2^-20 relative).
ACC_REL = 2.0 ** -12


def _validate_h(hq, hs, xe_rows, W1d):
    """GPU h codes/scales of one expert's rows against the oracle: equal, except
    where the oracle's h lies within the accumulation bound of an E4M3 rounding
    boundary (or its block maximum of a power of two); there the GPU's value
    must be one the interval [h - dh, h + dh] rounds to. Returns (mismatches,
    dequantised GPU h, dequantised oracle h)."""
    u = xe_rows @ W1d
    du = ACC_REL * (np.abs(xe_rows) @ np.abs(W1d)) + 2.0 ** -20 * np.abs(u)
    h = oracle.silu(u)
    dh = 1.1 * du + 2.0 ** -20 * np.abs(h)
    c_ref, s_ref = oracle.quantize_mx(h, axis=1)
    R, F = h.shape
    blk = lambda a: a.reshape(R, F // 32, 32)
    amax_lo = np.maximum(blk(np.abs(h) - dh).max(axis=2), 0.0)
    amax_hi = blk(np.abs(h) + dh).max(axis=2)
    e_lo = oracle.mx_scale_exponents(amax_lo) + 127
    e_hi = oracle.mx_scale_exponents(amax_hi) + 127
    assert ((hs == s_ref) | ((hs >= e_lo) & (hs <= e_hi))).all(), "h scale outside its rounding interval"
    X = np.repeat(np.ldexp(1.0, hs.astype(np.int64) - 127), 32, axis=1)
    vals = oracle.e4m3_values()
    v_lo = vals[oracle.e4m3_encode((h - dh) / X)] * X
    v_hi = vals[oracle.e4m3_encode((h + dh) / X)] * X
    v = vals[hq.astype(np.int64)] * X
    ok = (hq == c_ref) | ((v >= v_lo) & (v <= v_hi))
    assert ok.all(), f"{(~ok).sum()} h codes differ from the oracle away from a rounding boundary"
    return int((hq != c_ref).sum()), v, oracle.dequantize_mx(c_ref, s_ref, axis=1)


def _validate_layer(dev, I, tokens=None):
    """Step-wise MX path (quantise rows, permute, both products) and the one-call
    path on workload I; every check on the given tokens (default: all)."""
    d = gen.to_device(I, dev)
    W1q, W1s = moe.moe_quantize_mxfp8(d["W1"])
    W2q, W2s = moe.moe_quantize_mxfp8(d["W2"])
    ids, w = moe.moe_route(d["x"], d["Wr"], d["bias"], I.k, I.drop)
    _, off, row_token, inv = moe.moe_permute(d["x"], ids, w, I.E)
    hq, hs, y_perm = moe.moe_grouped_ffn_mxfp8(d["x"], row_token, off, W1q, W1s, W2q, W2s, I.F, I.k)
    y_steps = moe.moe_combine(y_perm, inv, w)
    y = moe.moe_forward_mxfp8(d["x"], d["Wr"], d["bias"], W1q, W1s, W2q, W2s, I.F, I.k, I.drop)
    y2 = moe.moe_forward_mxfp8(d["x"], d["Wr"], d["bias"], W1q, W1s, W2q, W2s, I.F, I.k, I.drop)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)  # deterministic
    A = int(off[-1].item())
    # the one-call path keeps y_perm as block-scaled fp16: within 2^-10 * max|y_perm| of the step-wise result,
    # and within the rounding bound element by element
    assert float((y - y_steps).abs().max()) <= 2.0 ** -10 * float(y_perm[:A].abs().max())
    if I.H % 32 == 0:
        eb = scaled16_bound(y_perm, A, inv, w, y_steps)
        assert bool(((y - y_steps).abs().double() <= eb).all()), "one-call y outside the fp16 rounding bound"

    r = oracle.route(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), I.k, I.drop)
    disp = oracle.dispatch(r.ids, r.keep, I.E)
    assert np.array_equal(ids.cpu().numpy(), r.ids)
    assert np.array_equal(off.cpu().numpy(), disp.offsets)
    assert np.array_equal(row_token.cpu().numpy()[:A], disp.row_token)
    tokens = np.arange(I.T) if tokens is None else np.asarray(tokens)
    x = I.f64(I.x)
    xe = oracle.dequantize_mx(*oracle.quantize_mx(x[tokens], axis=1), axis=1)
    W1, W2 = _mx_getter(I.W1, I.f64), _mx_getter(I.W2, I.f64)
    hq_n = hq.cpu().numpy().transpose(1, 0, 2).reshape(I.T * I.k, I.F)  # k-blocked [F/64][rows][64] -> [rows][F]
    hs_n = hs.cpu().numpy().transpose(1, 0, 2).reshape(I.T * I.k, I.F // 32)
    yp_n = y_perm.double().cpu().numpy()
    pos = {int(t): i for i, t in enumerate(tokens)}
    rows = sorted(int(disp.inv[t, j]) for t in tokens for j in range(I.k) if disp.inv[t, j] >= 0)
    yp_ref, extra, flips = {}, {}, 0
    by_expert = {}
    for rr in rows:
        by_expert.setdefault(int(np.searchsorted(disp.offsets, rr, side="right") - 1), []).append(rr)
    for e, rs in by_expert.items():
        xe_rows = xe[[pos[int(disp.row_token[rr])] for rr in rs]]
        n, v_gpu, v_ref = _validate_h(hq_n[rs], hs_n[rs], xe_rows, W1(e))
        flips += n
        ref = v_ref @ W2(e)
        # where h took a neighbouring code, y_perm may move by that code step through W2
        allow = np.abs(v_gpu - v_ref) @ np.abs(W2(e)) + ACC_REL * (np.abs(v_gpu) @ np.abs(W2(e)))
        for i, rr in enumerate(rs):
            yp_ref[rr], extra[rr] = ref[i], allow[i]
    ref_all = np.array([yp_ref[rr] for rr in rows])
    tol = Y_TOL * float(np.sqrt((ref_all ** 2).mean()))
    for rr in rows:
        assert np.all(np.abs(yp_n[rr] - yp_ref[rr]) <= tol + extra[rr]), f"y_perm row {rr}"
    # the layer output of the tokens: slot-order sum of the weighted rows
    y_n = y.double().cpu().numpy()
    y_ref = np.zeros((len(tokens), I.H))
    y_allow = np.zeros((len(tokens), I.H))
    for i, t in enumerate(tokens):
        for j in range(I.k):
            rr = int(disp.inv[t, j])
            if rr >= 0:
                y_ref[i] += r.w[t, j] * yp_ref[rr]
                y_allow[i] += r.w[t, j] * extra[rr]
    tol_y = Y_TOL * float(np.sqrt((y_ref ** 2).mean()))
    err = np.abs(y_n[tokens] - y_ref)
    assert np.all(err <= tol_y + y_allow), f"y: max-abs {err.max():.3e}, bar {tol_y:.3e} + flip allowance"
    return flips, len(rows) * I.F, float(err.max()) / float(np.sqrt((y_ref ** 2).mean()))


SMALL = [
    dict(T=300, H=256, F=256, E=6, k=2, zipf=1.2, seed=91),     # ~100 rows per expert, ragged tails
    dict(T=200, H=384, F=512, E=8, k=2, seed=92),                # 3 k-stages in W1, partial N tiles in W2
    dict(T=64, H=256, F=384, E=16, k=2, seed=93),                # few rows per expert, partial N tiles in W1
    dict(T=50, H=256, F=256, E=4, k=3, drop=0.1, seed=94),       # drop threshold
    dict(T=1, H=256, F=256, E=8, k=2, seed=95),                  # one token
]


@pytest.mark.parametrize("over", SMALL, ids=[f"small-{i}" for i in range(len(SMALL))])
def test_mx_layer_small(dev, over):
    I = gen.make_inputs("tiny", dtype="bf16", **over)
    _say(f"mx layer {over}")
    flips, n, rel = _validate_layer(dev, I)
    _say(f"  h codes at a rounding boundary: {flips} of {n}; y max-abs/rms {rel:.3e}")


@pytest.mark.parametrize("name", ["prefill", "decode"])
def test_mx_full_workload(dev, name):
    """Full-size MX layer, every token: h codes and scales, y_perm rows and y against the oracle."""
    I = gen.make_inputs(name)
    _say(f"mx full {name}: T={I.T} H={I.H} F={I.F} E={I.E} k={I.k}")
    flips, n, rel = _validate_layer(dev, I)
    _say(f"  {name}: h codes at a rounding boundary: {flips} of {n}; y max-abs/rms {rel:.3e} on all {I.T} tokens")
