"""Seeded random-shape GPU parity sweep.

Fifty-six layers with shapes drawn from fixed seeds (forty of any shape:
tokens, widths, expert counts, top-k, drop threshold, skewed router bias,
shared expert, fp32 or bf16; eight whose shared expert runs inside the routed
launches; eight on the 256x256 tiles with ragged widths) run through every
entry point the shape admits, each against the oracle:
* moe_forward and the step-wise route -> permute -> grouped_ffn -> combine;
* moe_forward_fp8 (weights-only fp8) when H, F are multiples of 64 and >= 128;
* moe_forward_mxfp8 (MX tokens and weights) when H, F are multiples of 128;
* moe_route_capacity when the router shape has the logits path.
Bars as in the dedicated tests: routing arrays bit-exact, weights within
2e-6, y within 2e-2 * rms (the MX layer with the near-boundary allowance of
tests/test_gpu_mx.py).
"""
import numpy as np
import pytest

import gen
import oracle
from tests.test_gpu_mx import _validate_layer

torch = pytest.importorskip("torch")
moe = pytest.importorskip("top_routing_grouped_gemm_amd")

pytestmark = pytest.mark.gpu

Y_TOL = 2e-2
W_TOL = 2e-6


def _draw_configs(n=20, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "f32" if i % 5 == 4 else "bf16"
        H = int(rng.choice([64, 128, 192, 256, 384, 512, 8 * int(rng.integers(1, 40))]))
        F = int(rng.choice([64, 128, 256, 384, 512, 8 * int(rng.integers(1, 60))]))
        E = int(rng.choice([1, 2, 4, 8, 16, 24, 40, 64, 128, 300]))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 3, 17, 64, 100, 257, 400, 1000, 2000]))
        drop = float(rng.choice([0.0, 0.0, 0.05, 0.1])) if k > 1 else 0.0
        drop = min(drop, 1.0 / k)
        zipf = float(rng.choice([0.0, 1.2])) if E >= 4 else 0.0
        Fs = int(rng.choice([0, 0, 0, 64, 136]))
        out.append(dict(T=T, H=H, F=F, E=E, k=k, drop=drop, zipf=zipf, Fs=Fs, dtype=dtype, seed=3000 + i))
    return out


def _draw_shared_merged(n=8, seed=2025):
    """bf16 layers whose shared expert runs as one more group of the routed launches: Fs == F, enough rows per
    expert for the large tiles (T*k/E >= 96), K and N multiples of 32, ragged T and F."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 4, 8]))
        k = int(rng.integers(1, min(E, 4) + 1))
        T = int(rng.choice([300, 513, 700, 1000, 2000]))
        if T * k // E < 96:
            T = 96 * E // k + 37
        H = int(32 * rng.integers(2, 17))
        F = int(32 * rng.integers(2, 21))
        drop = float(rng.choice([0.0, 0.1])) if k > 1 else 0.0
        out.append(dict(T=T, H=H, F=F, E=E, k=k, drop=min(drop, 1.0 / k), zipf=0.0, Fs=F, dtype="bf16",
                        seed=3100 + i))
    return out


def _draw_large_tiles(n=8, seed=2026):
    """bf16 layers on the 256x256 tiles (T*k/E >= 96) with widths that are multiples of 8 but not always of 32 or
    128: partial N-tiles and rows past each expert in every epilogue form the large tiles store through LDS (fp32
    y_perm, SiLU + bf16 h, block-scaled fp16 with word or byte scale stores)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 4, 6, 8]))
        k = int(rng.integers(1, min(E, 4) + 1))
        T = int(rng.integers(max(2, 100 * E // k), 2500))
        H = int(rng.choice([32 * int(rng.integers(2, 33)), 8 * int(rng.integers(8, 130))]))
        F = int(rng.choice([32 * int(rng.integers(2, 33)), 8 * int(rng.integers(8, 130))]))
        drop = float(rng.choice([0.0, 0.1])) if k > 1 else 0.0
        Fs = int(rng.choice([0, 0, 64]))
        out.append(dict(T=T, H=H, F=F, E=E, k=k, drop=min(drop, 1.0 / k), zipf=0.0, Fs=Fs, dtype="bf16",
                        seed=3200 + i))
    return out


CONFIGS = _draw_configs(40) + _draw_shared_merged(8) + _draw_large_tiles(8)


def _check_y(y_gpu, y_ref, tol=Y_TOL):
    rms = float(np.sqrt((y_ref ** 2).mean()))
    err = float(np.abs(y_gpu - y_ref).max())
    assert err <= tol * rms + 1e-30, f"max-abs error {err:.3e} > {tol} * rms {rms:.3e}"


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    return torch.device("cuda:0")


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: "T{T}-H{H}-F{F}-E{E}-k{k}-d{drop}-z{zipf}-s{Fs}-{dtype}".format(**c))
def test_random_layer(dev, cfg):
    print(f"case {cfg}", flush=True)
    I = gen.make_inputs("tiny", **cfg)
    d = gen.to_device(I, dev)
    T, H, F, E, k = I.T, I.H, I.F, I.E, I.k
    W1s, W2s = I.f64(I.W1s()) if I.Fs else None, I.f64(I.W2s()) if I.Fs else None
    ref = oracle.forward(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), I.f64(I.W1()), I.f64(I.W2()), k, I.drop, W1s, W2s)

    # one call
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    inv = torch.empty((T, k), dtype=torch.int32, device=dev)
    y = moe.moe_forward(d["x"], d["Wr"], d["bias"], d["W1"], d["W2"], k, I.drop, W1s=d["W1s"], W2s=d["W2s"],
                        topk_ids=ids, topk_w=w, expert_offsets=off, inv=inv)
    # step-wise
    ids2, w2 = moe.moe_route(d["x"], d["Wr"], d["bias"], k, I.drop)
    x_perm, off2, row_token, inv2 = moe.moe_permute(d["x"], ids2, w2, E)
    y_perm, y_sh = moe.moe_grouped_ffn(x_perm, off2, d["W1"], d["W2"], T, k, x=d["x"] if I.Fs else None,
                                       W1s=d["W1s"], W2s=d["W2s"])
    y2 = moe.moe_combine(y_perm, inv2, w2, y_sh)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ref.route.ids) and torch.equal(ids, ids2)
    assert np.abs(w.cpu().numpy() - ref.route.w).max() <= W_TOL and torch.equal(w, w2)
    assert np.array_equal(off.cpu().numpy(), ref.dispatch.offsets) and torch.equal(off, off2)
    assert np.array_equal(inv.cpu().numpy(), ref.dispatch.inv) and torch.equal(inv, inv2)
    A = int(ref.dispatch.offsets[-1])
    assert np.array_equal(row_token.cpu().numpy()[:A], ref.dispatch.row_token)
    _check_y(y.double().cpu().numpy(), ref.y)
    _check_y(y2.double().cpu().numpy(), ref.y)

    small = E * H * F <= 8 << 20
    bf16_plain = I.dtype == "bf16" and I.Fs == 0
    # weights-only fp8
    if bf16_plain and small and H % 64 == 0 and F % 64 == 0 and H >= 128 and F >= 128:
        W1q, s1 = moe.moe_quantize_fp8(d["W1"])
        W2q, s2 = moe.moe_quantize_fp8(d["W2"])
        y8 = moe.moe_forward_fp8(d["x"], d["Wr"], d["bias"], W1q, s1, W2q, s2, k, I.drop)
        torch.cuda.synchronize()
        c1, q1 = oracle.quantize_fp8(I.f64(I.W1()))
        c2, q2 = oracle.quantize_fp8(I.f64(I.W2()))
        r8 = oracle.forward(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), oracle.dequantize_fp8(c1, q1),
                            oracle.dequantize_fp8(c2, q2), k, I.drop)
        _check_y(y8.double().cpu().numpy(), r8.y)
        print("  fp8 weights: ok", flush=True)
    # MX tokens and weights
    if bf16_plain and small and H % 128 == 0 and F % 128 == 0:
        flips, n, rel = _validate_layer(dev, I)
        print(f"  MX: ok ({flips} of {n} h codes at a rounding boundary)", flush=True)
    # capacity-limited routing from x
    lib = moe.load_library()
    if I.dtype == "bf16" and lib.moe_route_capacity_workspace_bytes(T, H, E, moe.MOE_BF16) > 0:
        cap = oracle.capacity_slots(T, k, E, 1.2)
        if oracle.capacity_feasible(T, k, E, cap):
            r = oracle.route_capacity(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), k, I.drop, 1.2)
            if r.gap.min() >= 2e-4:  # decisions far from fp32 logit rounding
                idc, wc = moe.moe_route_capacity(d["x"], d["Wr"], d["bias"], k, I.drop, 1.2)
                torch.cuda.synchronize()
                assert np.array_equal(idc.cpu().numpy(), r.ids)
                assert np.abs(wc.cpu().numpy() - r.w).max() <= W_TOL
                print("  capacity routing: ok", flush=True)
