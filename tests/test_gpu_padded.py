"""GPU parity of the padded fixed-shape layout (the ablation of the ragged
grouped GEMM): every expert gets C rows, zero-padded.

Bar: the padded inverse map bit-exact against the one derived from the
oracle's dispatch; y within 2e-2 * rms of the oracle; with C at least the
largest expert count, y equal to the ragged path's within fp32 rounding.
"""
import numpy as np
import pytest

import gen
import oracle

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


def _expected_inv_pad(r, disp, E, C):
    T, k = r.ids.shape
    out = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            row = disp.inv[t, j]
            if row >= 0:
                e = r.ids[t, j]
                i = row - disp.offsets[e]
                if i < C:
                    out[t, j] = e * C + i
    return out


@pytest.mark.parametrize("name,over,c_shrink", [
    ("decode", {}, 0),                                                                       # C = largest count
    ("tiny", {"T": 300, "H": 128, "F": 192, "E": 6, "k": 2, "dtype": "bf16", "seed": 51, "zipf": 1.2}, 0),
    ("tiny", {"T": 300, "H": 128, "F": 192, "E": 6, "k": 2, "dtype": "bf16", "seed": 51, "zipf": 1.2}, 40),  # drops
])
def test_padded_layer(dev, name, over, c_shrink):
    I = gen.make_inputs(name, **over)
    d = gen.to_device(I, dev)
    ids, w = moe.moe_route(d["x"], d["Wr"], d["bias"], I.k, I.drop)
    x_perm, off, row_token, inv = moe.moe_permute(d["x"], ids, w, I.E)
    y_perm, _ = moe.moe_grouped_ffn(x_perm, off, d["W1"], d["W2"], I.T, I.k)
    y_ragged = moe.moe_combine(y_perm, inv, w)
    torch.cuda.synchronize()
    counts = (off[1:] - off[:-1]).cpu().numpy()
    C = int(counts.max()) - c_shrink
    x_pad, inv_pad = moe.moe_pad_dispatch(d["x"], ids, off, row_token, inv, I.E, C)
    y_pad = moe.moe_grouped_ffn_padded(x_pad, d["W1"], d["W2"], C)
    y = moe.moe_combine(y_pad, inv_pad, w)
    torch.cuda.synchronize()

    r = oracle.route(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), I.k, I.drop)
    disp = oracle.dispatch(r.ids, r.keep, I.E)
    exp_inv = _expected_inv_pad(r, disp, I.E, C)
    assert np.array_equal(inv_pad.cpu().numpy(), exp_inv)
    # the padding rows are zero
    xp = x_pad.view(I.E, C, I.H).float().cpu().numpy()
    for e in range(I.E):
        assert not xp[e, min(C, counts[e]):].any()
    # oracle: the layer with the slots beyond C removed (their weight is not renormalised)
    yp = oracle.grouped_ffn(I.f64(I.x)[disp.row_token], disp.offsets, lambda e: I.f64(I.W1(e, e + 1)[0]),
                            lambda e: I.f64(I.W2(e, e + 1)[0]))
    inv_kept = np.where(exp_inv >= 0, disp.inv, -1)
    y_ref = oracle.combine(yp, inv_kept, r.w)
    err = np.abs(y.double().cpu().numpy() - y_ref).max() / np.sqrt((y_ref ** 2).mean())
    assert err <= Y_TOL
    if c_shrink == 0:
        assert float((y - y_ragged).abs().max()) <= 1e-5 * float(y_ragged.abs().max())
