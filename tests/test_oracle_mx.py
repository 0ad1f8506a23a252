"""Pins of the oracle's MX fp8 quantisation (CPU only).

Reading of page 1 ("MoE大模型的智能调度…", www.jsqmd.com/news/1091713),
section 4.1 (experts in 8 bits) extended to the activations, on the MI355X fp8
matrix cores: the OCP MX block format with E4M3 elements -- 32 consecutive
values along a product's reduction axis share a power-of-two scale
2^(floor(log2 amax) - 8), stored as a biased exponent byte. Pins fixed
outside the oracle's own code:

* hand values of the shared exponent;
* the scale characterised independently: the unique power of two X with
  amax / X in [256, 512);
* codes equal a per-element brute-force E4M3 encoding of V / X;
* the error bound of the dequantised values (half an E4M3 step, or the clamp
  at 448 X);
* blocks lie along the requested axis, 32 wide;
* the MX expert re-quantises its SiLU output along F: its difference from the
  unquantised expert is non-zero and within the bound that h's quantisation
  error implies;
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
from tests.test_oracle_fp8 import brute_force_encode  # noqa: E402


def _block_scales(V, axis):
    """X per element: the power of two with amax/X in [256, 512), found by search."""
    Vm = np.moveaxis(np.asarray(V, dtype=np.float64), axis, -1)
    blocks = Vm.reshape(Vm.shape[:-1] + (Vm.shape[-1] // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    X = np.ones_like(amax)
    for idx in np.ndindex(amax.shape):
        a = amax[idx]
        if a == 0:
            continue
        p = 0
        while a / 2.0 ** p >= 512:
            p += 1
        while a / 2.0 ** p < 256:
            p -= 1
        X[idx] = 2.0 ** p
    Xe = np.repeat(X, 32, axis=-1)
    return np.moveaxis(Xe, -1, axis)


# ------------------------------------------------------------------- pins --
def check_exponent_values():
    a = np.array([448.0, 256.0, 255.99, 1.0, 0.75, 512.0, 0.0, 2.0 ** -140, 2.0 ** 200, 3.0 * 2 ** -20])
    want = [0, 0, -1, -8, -9, 1, 0, -127, 127, -27]
    assert oracle.mx_scale_exponents(a).tolist() == want


def check_scale_characterisation():
    rng = np.random.default_rng(31)
    V = (rng.standard_normal((6, 128)) * np.exp(rng.uniform(-6, 6, (6, 1)))).astype(np.float32)
    V[2, 32:64] = 0.0
    codes, sb = oracle.quantize_mx(V, axis=1)
    X = _block_scales(V, 1)
    got = np.repeat(np.ldexp(1.0, sb.astype(np.int64) - 127), 32, axis=1)
    assert np.array_equal(got, X)
    assert sb.shape == (6, 4) and sb.dtype == np.uint8


def check_codes_brute_force():
    rng = np.random.default_rng(32)
    V = (rng.standard_normal((3, 64)) * np.exp(rng.uniform(-4, 4, (3, 64)))).astype(np.float32)
    codes, sb = oracle.quantize_mx(V, axis=1)
    X = _block_scales(V, 1)
    assert np.array_equal(codes, brute_force_encode(V.astype(np.float64) / X))


def check_error_bound():
    rng = np.random.default_rng(33)
    V = (rng.standard_normal((8, 96)) * np.exp(rng.uniform(-3, 3, (8, 96)))).astype(np.float32)
    codes, sb = oracle.quantize_mx(V, axis=1)
    deq = oracle.dequantize_mx(codes, sb, axis=1)
    X = _block_scales(V, 1)
    r = np.abs(V.astype(np.float64)) / X
    bound = X * np.maximum(np.maximum(r * 2.0 ** -4, 2.0 ** -10), r - 448.0)
    assert np.all(np.abs(deq - V) <= bound)
    # the block maximum is encoded within the clamp: its code is 0x7E (448) or within an E4M3 step of it
    assert ((codes & 0x7F) <= 0x7E).all()


def check_axis_and_block_width():
    rng = np.random.default_rng(34)
    W = rng.standard_normal((2, 64, 8)).astype(np.float32)   # blocks along axis 1 (the reduction axis K)
    c0, s0 = oracle.quantize_mx(W, axis=1)
    assert s0.shape == (2, 2, 8)
    W2 = W.copy()
    W2[1, 40, 3] = 1000.0                                      # block (e=1, kb=1, n=3) only
    c1, s1 = oracle.quantize_mx(W2, axis=1)
    diff = s1 != s0
    assert diff.sum() == 1 and diff[1, 1, 3]
    changed = np.argwhere((c1 != c0).any(axis=1))
    assert all((e, n) == (1, 3) for e, n in changed)
    assert (c1[1, 32:64, 3] != c0[1, 32:64, 3]).any() and np.array_equal(c1[1, :32, 3], c0[1, :32, 3])


def check_mx_expert_requantises_h():
    rng = np.random.default_rng(35)
    rows = rng.standard_normal((5, 64))
    W1 = rng.standard_normal((64, 96)) / 8
    W2 = rng.standard_normal((96, 64)) / 10
    y_mx = oracle.expert_ffn_mx(rows, W1, W2)
    y = oracle.expert_ffn(rows, W1, W2)
    h = oracle.silu(rows @ W1)
    X = _block_scales(h, 1)
    r = np.abs(h) / X
    dh = X * np.maximum(np.maximum(r * 2.0 ** -4, 2.0 ** -10), r - 448.0)
    bound = dh @ np.abs(W2)
    d = np.abs(y_mx - y)
    assert d.max() > 0
    assert np.all(d <= bound * (1 + 1e-9) + 1e-12)


PINS = [check_exponent_values, check_scale_characterisation, check_codes_brute_force, check_error_bound,
        check_axis_and_block_width, check_mx_expert_requantises_h]


@pytest.mark.parametrize("check", PINS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


# --------------------------------------------------------- planted mistakes --
_orig_exp = moe_oracle.mx_scale_exponents
_orig_quant = moe_oracle.quantize_mx
_orig_ffn = moe_oracle.expert_ffn_mx


def _mut_emax7(amax):
    return np.clip(_orig_exp(amax) + 1, -127, 127)  # the E4M3 maximum exponent taken as 7


def _mut_ceil(amax):
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        x = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1))) - 8, 0)
    return np.clip(x, -127, 127).astype(np.int64)


def _mut_block16(V, axis):
    V32 = np.asarray(V, dtype=np.float32)
    Vm = np.moveaxis(V32, axis, -1)
    n = Vm.shape[-1]
    blocks = Vm.reshape(Vm.shape[:-1] + (n // 16, 16))
    xexp = moe_oracle.mx_scale_exponents(np.abs(blocks).max(axis=-1))
    codes = moe_oracle.e4m3_encode(blocks.astype(np.float64) * np.ldexp(1.0, -xexp)[..., None]).reshape(Vm.shape)
    xexp = xexp[..., ::2]
    return np.moveaxis(codes, -1, axis), np.moveaxis((xexp + 127).astype(np.uint8), -1, axis)


def _mut_last_axis(V, axis):
    return _orig_quant(V, np.ndim(V) - 1)  # blocks always along the last axis


def _mut_no_requant(rows, W1e, W2e):
    return moe_oracle.silu(rows @ W1e) @ W2e


MUTATIONS = [("mx_scale_exponents", _mut_emax7), ("mx_scale_exponents", _mut_ceil), ("quantize_mx", _mut_block16),
             ("quantize_mx", _mut_last_axis), ("expert_ffn_mx", _mut_no_requant)]


@pytest.mark.parametrize("name,mutation", MUTATIONS, ids=lambda v: v if isinstance(v, str) else v.__name__)
def test_planted_mistakes(name, mutation, monkeypatch):
    """Every planted bug in the oracle's MX quantisation makes at least one pin fail."""
    failed = []
    with monkeypatch.context() as mp:
        mp.setattr(moe_oracle, name, mutation)
        mp.setattr(oracle, name, mutation)
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError, IndexError):
                failed.append(pin.__name__)
    assert failed, f"{mutation.__name__} survived every pin"
