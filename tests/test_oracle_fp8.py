"""Pins of the oracle's low-precision expert weights (CPU only).

Page 1 ("MoE大模型的智能调度…", www.jsqmd.com/news/1091713), section 4.1
(model loading and memory budget): the resident experts' FFN weights are
stored in 8 bits. The oracle reads this, for MI355X, as OCP fp8 e4m3 codes
with one fp32 scale per expert and output column (max |W| / 448), codes by
round-to-nearest-even of W / scale. These pins check it against things fixed
outside its own code:

* code values the OCP 8-bit floating-point format fixes (bias 7, subnormals,
  NaN at 0x7F/0xFF, largest finite 448);
* a library special case: PyTorch's float8_e4m3fn bit reinterpretation and
  its float32 -> e4m3 conversion (inside the finite range);
* brute force: the nearest of all 127 magnitudes, ties to the even code;
* round trips, midpoints and the half-ulp error bound of the quantised
  weights, the column maximum landing on +-448, all-zero columns;
* planted mistakes in the oracle, each caught by at least one of the above.
"""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from oracle import moe_oracle  # noqa: E402


def brute_force_encode(x):
    """Nearest of the 127 non-negative finite magnitudes by exhaustive search;
    on a tie the even code; the sign bit copied from x."""
    mags = [c for c in range(0x7F)]
    vals = {}
    for c in mags:  # values written out from the format: bias 7, subnormal exponent 0
        e, m = c >> 3, c & 7
        vals[c] = m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10)
    out = []
    for v in np.asarray(x, dtype=np.float64).ravel():
        a = abs(float(v))
        best, bd = None, None
        for c in mags:
            d = abs(a - vals[c])
            if bd is None or d < bd or (d == bd and c % 2 == 0):
                best, bd = c, d
        out.append(best | (0x80 if np.signbit(v) else 0))
    return np.array(out, dtype=np.uint8).reshape(np.shape(x))


# ------------------------------------------------------------------- pins --
def check_code_values():
    v = oracle.e4m3_values()
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 15 * 2.0 ** -9,
             0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0x78: 256.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -2.0 ** -9}
    for c, want in fixed.items():
        assert v[c] == want, (hex(c), v[c], want)
    assert np.signbit(v[0x80]) and v[0x80] == 0.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[0x80:0xFF], -pos)


def check_torch_special_case():
    torch = pytest.importorskip("torch")
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    v = oracle.e4m3_values()
    assert np.array_equal(np.isnan(lib), np.isnan(v))
    assert np.array_equal(lib[~np.isnan(lib)], v[~np.isnan(v)])
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-14, 6, 200000))).astype(np.float32)
    x = x[np.abs(x) < 464].astype(np.float32)  # torch maps values past 464 to NaN (no saturation)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), ref)


def check_brute_force():
    rng = np.random.default_rng(22)
    x = rng.standard_normal(1500) * np.exp(rng.uniform(-12, 7, 1500))
    x = np.concatenate([x, [0.0, -0.0, 448.0, 449.0, 464.0, 480.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -10,
                            2.0 ** -11, -2.0 ** -10]])
    assert np.array_equal(oracle.e4m3_encode(x), brute_force_encode(x))


def check_round_trip_and_midpoints():
    v = oracle.e4m3_values()
    codes = np.array([c for c in range(256) if np.isfinite(v[c])])
    assert np.array_equal(oracle.e4m3_encode(v[codes]), codes.astype(np.uint8))
    pos = v[:0x7F]
    mid = (pos[:-1] + pos[1:]) / 2  # exact in float64: a tie between codes c and c+1
    got = oracle.e4m3_encode(mid).astype(int)
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    # just off the midpoint the nearer code wins
    assert np.array_equal(oracle.e4m3_encode(np.nextafter(mid, 0)).astype(int), lo)
    assert np.array_equal(oracle.e4m3_encode(np.nextafter(mid, 1e9)).astype(int), lo + 1)


def check_quantize_properties():
    rng = np.random.default_rng(23)
    E, K, N = 3, 64, 40
    W = (rng.standard_normal((E, K, N)) * np.exp(rng.uniform(-3, 3, (1, 1, N)))).astype(np.float32)
    W[1, :, 7] = 0.0  # an all-zero column
    codes, s = oracle.quantize_fp8(W)
    assert codes.shape == (E, K, N) and codes.dtype == np.uint8 and s.shape == (E, N) and s.dtype == np.float32
    amax = np.abs(W).max(axis=1)
    want_s = (amax / np.float32(448)).astype(np.float32)
    want_s[want_s == 0] = 1
    assert np.array_equal(s, want_s)
    assert s[1, 7] == 1.0 and not codes[1, :, 7].any()
    # each column's largest magnitude lands on +-448
    for e in range(E):
        for n in range(N):
            if amax[e, n] == 0:
                continue
            kk = int(np.argmax(np.abs(W[e, :, n])))
            assert codes[e, kk, n] & 0x7F == 0x7E
    # half-ulp error bound of the dequantised weights (3 mantissa bits; subnormal step 2^-9)
    deq = oracle.dequantize_fp8(codes, s)
    r = np.abs(W.astype(np.float64)) / s.astype(np.float64)[:, None, :]
    bound = s.astype(np.float64)[:, None, :] * (np.maximum(r * 2.0 ** -4, 2.0 ** -10) + r * 2.0 ** -22)
    assert np.all(np.abs(deq - W) <= bound)
    # bf16 input gives the same codes as its exact float32 widening
    Wb = (W.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    c2, s2 = oracle.quantize_fp8(Wb.astype(np.float64))
    c3, s3 = oracle.quantize_fp8(Wb)
    assert np.array_equal(c2, c3) and np.array_equal(s2, s3)


def check_scale_is_per_expert_and_column():
    rng = np.random.default_rng(24)
    W = rng.standard_normal((2, 32, 16)).astype(np.float32)
    c0, s0 = oracle.quantize_fp8(W)
    W2 = W.copy()
    W2[1, :, 5] *= 1024  # exact power of two: only that column's scale moves, its codes stay
    c1, s1 = oracle.quantize_fp8(W2)
    assert np.array_equal(c0, c1)
    assert s1[1, 5] == s0[1, 5] * 1024
    mask = np.ones_like(s0, dtype=bool)
    mask[1, 5] = False
    assert np.array_equal(s0[mask], s1[mask])


PINS = [check_code_values, check_torch_special_case, check_brute_force, check_round_trip_and_midpoints,
        check_quantize_properties, check_scale_is_per_expert_and_column]


@pytest.mark.parametrize("check", PINS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


# --------------------------------------------------------- planted mistakes --
_orig_values = moe_oracle.e4m3_values
_orig_encode = moe_oracle.e4m3_encode
_orig_quant = moe_oracle.quantize_fp8


def _mut_bias8():
    v = _orig_values()
    return v / 2  # exponent bias 8 instead of 7


def _mut_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    c = _orig_encode(x).astype(np.int64)
    v = _orig_values()[:0x7F]
    m = c & 0x7F
    nxt = np.minimum(m + 1, 0x7E)
    tie_above = (np.minimum(np.abs(x), 448.0) == (v[m] + v[nxt]) / 2) & (nxt != m)
    return np.where(tie_above, (c & 0x80) | nxt, c).astype(np.uint8)  # a tie goes up, even or not


def _mut_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    v = _orig_values()[:0x7F]
    a = np.minimum(np.abs(x), 448.0)
    c = np.searchsorted(v, a, side="right") - 1  # largest magnitude <= |x|
    return (c | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def _mut_row_scale(W):
    W32 = np.asarray(W, dtype=np.float32)
    amax = np.abs(W32).max(axis=2)  # per row instead of per output column
    s = (amax / np.float32(448)).astype(np.float32)
    s = np.where(s == 0, np.float32(1), s).astype(np.float32)
    codes = moe_oracle.e4m3_encode((W32 / s[:, :, None]).astype(np.float32))
    return codes, np.broadcast_to(s.max(axis=1, keepdims=True), (W32.shape[0], W32.shape[2])).copy()


def _mut_fnuz_max(W):
    W32 = np.asarray(W, dtype=np.float32)
    s = (np.abs(W32).max(axis=1) / np.float32(240)).astype(np.float32)  # the e4m3 "fnuz" maximum
    s = np.where(s == 0, np.float32(1), s).astype(np.float32)
    return moe_oracle.e4m3_encode((W32 / s[:, None, :]).astype(np.float32)), s


MUTATIONS = [("e4m3_values", _mut_bias8), ("e4m3_encode", _mut_ties_away), ("e4m3_encode", _mut_truncate),
             ("quantize_fp8", _mut_row_scale), ("quantize_fp8", _mut_fnuz_max)]


@pytest.mark.parametrize("name,mutation", MUTATIONS, ids=lambda v: v if isinstance(v, str) else v.__name__)
def test_planted_mistakes(name, mutation, monkeypatch):
    """Every planted bug in the oracle's fp8 quantisation makes at least one pin fail."""
    failed = []
    with monkeypatch.context() as mp:
        mp.setattr(moe_oracle, name, mutation)
        mp.setattr(oracle, name, mutation)
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                failed.append(pin.__name__)
    assert failed, f"{mutation.__name__} survived every pin"
