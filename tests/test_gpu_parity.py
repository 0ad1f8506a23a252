"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bar: expert ids, expert offsets, row order (row_token), inverse map and the
permuted rows are bit-exact; routing weights within 2e-6; layer output y
within max-abs 2e-2 * rms(y_oracle) (bf16 operands, fp32 accumulation).
Full-size workloads compare every routing array and every token of y_perm and
y (one-call and step-wise) with the oracle's whole layer.
"""
import numpy as np
import pytest

import gen
import oracle
from tests.scaled16 import scaled16_bound
from tests.test_oracle import worked_example_inputs, _golden

torch = pytest.importorskip("torch")
moe = pytest.importorskip("top_routing_grouped_gemm_amd")

pytestmark = pytest.mark.gpu

W_TOL = 2e-6
Y_TOL = 2e-2


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def run_steps(d, I, dev, out_dtype=torch.float32):
    """route -> permute -> grouped_ffn -> combine through the step-wise entry points."""
    T, k, E = I.T, I.k, I.E
    ids, w = moe.moe_route(d["x"], d["Wr"], d["bias"], k, I.drop)
    x_perm, off, row_token, inv = moe.moe_permute(d["x"], ids, w, E)
    y_perm, y_sh = moe.moe_grouped_ffn(x_perm, off, d["W1"], d["W2"], T, k, x=d["x"] if I.Fs else None,
                                       W1s=d["W1s"], W2s=d["W2s"])
    y = moe.moe_combine(y_perm, inv, w, y_sh, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return dict(ids=ids, w=w, x_perm=x_perm, off=off, row_token=row_token, inv=inv, y_perm=y_perm, y_sh=y_sh, y=y)


def check_routing(g, ref_route, ref_disp, x_storage=None, I=None):
    ids = g["ids"].cpu().numpy()
    w = g["w"].cpu().numpy().astype(np.float64)
    assert np.array_equal(ids, ref_route.ids), "expert ids differ"
    assert np.abs(w - ref_route.w).max() <= W_TOL, "routing weights differ"
    assert np.array_equal(w == 0.0, ~ref_route.keep), "dropped slots differ"
    off = g["off"].cpu().numpy()
    assert np.array_equal(off, ref_disp.offsets), "expert offsets differ"
    A = int(off[-1])
    assert np.array_equal(g["row_token"].cpu().numpy()[:A], ref_disp.row_token), "row order differs"
    assert np.array_equal(g["inv"].cpu().numpy(), ref_disp.inv), "inverse map differs"
    if x_storage is not None:
        xp = g["x_perm"][:A].cpu()
        xp = xp.view(torch.int16).numpy().view(np.uint16) if xp.dtype == torch.bfloat16 else xp.numpy()
        assert np.array_equal(xp, x_storage[ref_disp.row_token]), "permuted rows differ"


def check_y(y_gpu, y_ref, tol=Y_TOL):
    rms = float(np.sqrt((y_ref ** 2).mean()))
    err = float(np.abs(y_gpu - y_ref).max())
    assert err <= tol * rms, f"max-abs error {err:.3e} > {tol} * rms {rms:.3e}"
    return err / rms


# ------------------------------------------------------ worked example --
def _we_device(dev, pad_to=8):
    x, Wr, _, k = worked_example_inputs()
    T, E = x.shape
    xp = np.zeros((T, pad_to), dtype=np.float32)
    xp[:, :E] = x
    Wrp = np.zeros((pad_to, E), dtype=np.float32)
    Wrp[:E] = Wr
    return torch.from_numpy(xp).to(dev), torch.from_numpy(Wrp).to(dev), k, E


@pytest.mark.parametrize("drop", [0.0, 0.25])
def test_worked_example(dev, drop):
    g = _golden()
    exp = g["derived"] if drop == 0.0 else dict(g["derived"], **g["drop_case"])
    x, Wr, k, E = _we_device(dev)
    ids, w = moe.moe_route(x, Wr, None, k, drop)
    x_perm, off, row_token, inv = moe.moe_permute(x, ids, w, E)
    torch.cuda.synchronize()
    assert ids.cpu().tolist() == exp["topk_ids"]
    assert np.abs(w.cpu().numpy() - np.array(exp["topk_w"])).max() <= 1e-6
    assert off.cpu().tolist() == exp["offsets"]
    A = exp["offsets"][-1]
    assert row_token.cpu().tolist()[:A] == exp["row_token"]
    assert inv.cpu().tolist() == exp["inv"]
    # combine with unit-vector expert rows: y[t] spells out (row, weight) pairs
    y_perm = torch.zeros((8, 8), dtype=torch.float32, device=dev)
    y_perm[:A] = torch.eye(8, device=dev)[:A]
    y = moe.moe_combine(y_perm, inv, w).cpu().numpy()
    want = np.zeros((4, 8))
    for t in range(4):
        for j in range(2):
            r = exp["inv"][t][j]
            if r >= 0:
                want[t, r] += exp["topk_w"][t][j]
    assert np.abs(y - want).max() <= 1e-6


# --------------------------------------------------------- small layers --
SMALL = [
    ("tiny", {}),
    ("tiny", {"dtype": "bf16", "seed": 77}),
    ("tiny", {"T": 37, "H": 64, "F": 96, "E": 8, "k": 3, "dtype": "bf16", "seed": 78}),     # ragged tails
    ("tiny", {"T": 300, "H": 136, "F": 200, "E": 16, "k": 4, "dtype": "bf16", "seed": 79}),
    ("tiny", {"T": 200, "H": 128, "F": 136, "E": 6, "k": 2, "dtype": "bf16", "seed": 80, "drop": 0.3,
              "zipf": 1.2}),
    ("tiny", {"T": 1, "H": 64, "F": 64, "E": 8, "k": 2, "dtype": "bf16", "seed": 81}),      # one token
    ("tiny", {"T": 50, "H": 64, "F": 64, "E": 5, "k": 5, "dtype": "f32", "seed": 82}),      # k == E
    ("tiny", {"T": 40, "H": 64, "F": 64, "E": 1, "k": 1, "dtype": "bf16", "seed": 83}),     # single expert
    ("tiny", {"T": 64, "H": 64, "F": 128, "E": 4, "k": 2, "dtype": "bf16", "seed": 84, "Fs": 64}),  # shared
    ("tiny", {"T": 90, "H": 72, "F": 40, "E": 12, "k": 2, "dtype": "f32", "seed": 85, "Fs": 24, "drop": 0.2}),
    ("tiny", {"T": 520, "H": 64, "F": 64, "E": 300, "k": 6, "dtype": "bf16", "seed": 86}),  # E > 256, E%8 != 0 rows
    # the size limits: E = 1024 experts, top-32
    ("tiny", {"T": 40, "H": 64, "F": 64, "E": 1024, "k": 32, "dtype": "bf16", "seed": 96}),
    ("tiny", {"T": 24, "H": 64, "F": 40, "E": 1024, "k": 32, "dtype": "f32", "seed": 97, "drop": 0.02}),
    # large-tile (direct-to-LDS) path: K % 64 == 0, >= 96 rows per expert, partial N tiles
    ("tiny", {"T": 700, "H": 128, "F": 192, "E": 5, "k": 2, "dtype": "bf16", "seed": 87}),
    ("tiny", {"T": 300, "H": 256, "F": 320, "E": 4, "k": 2, "dtype": "bf16", "seed": 88, "Fs": 192}),
    # Fs == F on the large tiles: the shared expert is one more group of the routed launches (ragged last
    # shared M-tile, partial N tile; with drop)
    ("tiny", {"T": 300, "H": 256, "F": 320, "E": 4, "k": 2, "dtype": "bf16", "seed": 90, "Fs": 320}),
    ("tiny", {"T": 520, "H": 128, "F": 256, "E": 3, "k": 2, "dtype": "bf16", "seed": 91, "Fs": 256, "drop": 0.2}),
    ("tiny", {"T": 1100, "H": 192, "F": 128, "E": 8, "k": 3, "dtype": "bf16", "seed": 89, "drop": 0.2,
              "zipf": 1.2}),
]


@pytest.mark.parametrize("name,over", SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SMALL)])
def test_small_layers(dev, name, over):
    I = gen.make_inputs(name, **over)
    _say(f"case {name} {over}")
    d = gen.to_device(I, dev)
    g = run_steps(d, I, dev)
    W1s, W2s = I.f64(I.W1s()), I.f64(I.W2s())
    ref = oracle.forward(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), I.f64(I.W1()), I.f64(I.W2()), I.k, I.drop, W1s, W2s)
    check_routing(g, ref.route, ref.dispatch, I.x)
    A = int(ref.dispatch.offsets[-1])
    check_y(g["y_perm"][:A].double().cpu().numpy(), ref.y_perm)
    check_y(g["y"].double().cpu().numpy(), ref.y)
    # the one-call path: same bar against the oracle, and against the step-wise path within the one extra
    # rounding it may take (y_perm kept as block-scaled fp16 inside moe_forward), element by element
    y2 = moe.moe_forward(d["x"], d["Wr"], d["bias"], d["W1"], d["W2"], I.k, I.drop, W1s=d["W1s"], W2s=d["W2s"])
    torch.cuda.synchronize()
    check_y(y2.double().cpu().numpy(), ref.y)
    if I.H % 32 == 0:
        bound = scaled16_bound(g["y_perm"], A, g["inv"], g["w"], g["y"])
        assert bool(((y2 - g["y"]).abs().double() <= bound).all()), "one-call y outside the fp16 rounding bound"
    else:  # no whole 32-column blocks: y_perm stays fp32 (coarse check)
        bound = 2.0 ** -10 * float(g["y_perm"][:A].abs().max()) if A else 0.0
        assert float((y2 - g["y"]).abs().max()) <= bound


@pytest.mark.parametrize("T,H,E,k,drop,zipf", [
    (32, 512, 128, 8, 0.0, 0.0),      # few tokens: H loop split across workgroups, ordered reduction
    (100, 256, 64, 4, 0.0, 0.0),
    (3000, 128, 256, 8, 0.0, 0.0),    # one pass, E = 256
    (50, 64, 16, 2, 0.0, 0.0),
    (77, 192, 24, 3, 0.1, 1.2),       # E < 32 padded columns, bias, drop
    (1, 1024, 40, 5, 0.0, 0.0),       # one token, many splits
    (8, 2048, 128, 8, 0.0, 0.0),      # 32 splits: one workgroup per token in the reduction, eight loads a thread
    (2, 4096, 32, 4, 0.0, 0.0),       # 64 splits over 32 padded expert columns
])
def test_router_paths(dev, T, H, E, k, drop, zipf):
    I = gen.make_inputs("tiny", T=T, H=H, F=64, E=E, k=k, dtype="bf16", seed=95 + T, drop=drop, zipf=zipf)
    d = gen.to_device(I, dev)
    ids, w = moe.moe_route(d["x"], d["Wr"], d["bias"], I.k, I.drop)
    ids2, w2 = moe.moe_route(d["x"], d["Wr"], d["bias"], I.k, I.drop)
    torch.cuda.synchronize()
    r = oracle.route(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), I.k, I.drop)
    assert np.array_equal(ids.cpu().numpy(), r.ids)
    assert np.abs(w.cpu().numpy() - r.w).max() <= W_TOL
    assert torch.equal(ids, ids2) and torch.equal(w, w2)


def test_router_odd_expert_count(dev):
    """E % 8 != 0 takes the scalar Wr path of the bf16 router."""
    I = gen.make_inputs("tiny", T=70, H=64, F=64, E=13, k=3, dtype="bf16", seed=90)
    d = gen.to_device(I, dev)
    ids, w = moe.moe_route(d["x"], d["Wr"], None, I.k)
    torch.cuda.synchronize()
    r = oracle.route(I.f64(I.x), I.f64(I.Wr), None, I.k)
    assert np.array_equal(ids.cpu().numpy(), r.ids)
    assert np.abs(w.cpu().numpy() - r.w).max() <= W_TOL


# ------------------------------------------------- stage tests, ragged --
@pytest.mark.parametrize("counts", [
    [0, 1, 16, 17, 0, 64, 65, 128, 129, 3],      # empty, 1 row, tile edges of every tile shape
    [0, 0, 0, 700, 0],                           # all rows to one expert
    [1] * 40,                                    # decode-like: one row per expert
    [0, 0, 0, 0, 0, 0, 0, 5],                    # only the last expert
    [130, 0, 257, 1, 128, 129, 0, 300],          # large tiles: 128-row edges, partial and single rows
])
@pytest.mark.parametrize("dtype,H,F", [("bf16", 72, 136), ("f32", 72, 136), ("bf16", 128, 320)])
def test_grouped_ffn_ragged(dev, counts, dtype, H, F):
    """Oracle-fed grouped FFN: x_perm and offsets built on the host, y_perm vs the oracle's grouped FFN."""
    E = len(counts)
    A = sum(counts)
    seed = 500 + A + E
    x = gen.normal(seed, 1, A * H, 1.0, dtype).reshape(A, H)
    W1 = gen.normal(seed, 3, E * H * F, 1 / np.sqrt(H), dtype).reshape(E, H, F)
    W2 = gen.normal(seed, 4, E * F * H, 1 / np.sqrt(F), dtype).reshape(E, F, H)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    k = 1
    T = A  # capacity rows = T*k
    tx = gen.storage_to_torch(x, dtype).to(dev)
    tW1 = gen.storage_to_torch(W1, dtype).to(dev)
    tW2 = gen.storage_to_torch(W2, dtype).to(dev)
    toff = torch.from_numpy(off).to(dev)
    y_perm, _ = moe.moe_grouped_ffn(tx, toff, tW1, tW2, T, k)
    torch.cuda.synchronize()
    ref = oracle.grouped_ffn(gen.to_f64(x, dtype), off, gen.to_f64(W1, dtype), gen.to_f64(W2, dtype))
    check_y(y_perm.double().cpu().numpy(), ref)


def test_combine_oracle_fed(dev):
    """Oracle-fed combine: inv, weights and y_perm from the oracle; y must match to fp32 rounding."""
    I = gen.make_inputs("tiny", T=123, H=64, F=32, E=9, k=3, dtype="f32", seed=91, drop=0.2)
    ref = oracle.forward(I.f64(I.x), I.f64(I.Wr), None, I.f64(I.W1()), I.f64(I.W2()), I.k, I.drop)
    A = int(ref.dispatch.offsets[-1])
    yp = torch.zeros((I.T * I.k, I.H), dtype=torch.float32)
    yp[:A] = torch.from_numpy(ref.y_perm)
    y = moe.moe_combine(yp.to(dev), torch.from_numpy(ref.dispatch.inv.astype(np.int32)).to(dev),
                        torch.from_numpy(ref.route.w.astype(np.float32)).to(dev))
    torch.cuda.synchronize()
    assert np.abs(y.double().cpu().numpy() - ref.y).max() <= 1e-5 * np.abs(ref.y).max()


@pytest.mark.parametrize("T,E", [
    (777, 37),     # 3108 assignments: the two-pass dispatch (count+rank, finalize)
    (9000, 1000),  # 36 chunks x 1000 experts > 32768 counts: count / scan / index kernels
    (256, 37),     # 1024 assignments: the single-workgroup dispatch, at its limit
    (257, 1000),   # 1028 assignments just past it, E near the maximum
    (200, 1000),   # 800 assignments over 1000 experts in one workgroup
])
def test_permute_oracle_fed(dev, T, E):
    """Oracle-fed permute: ids/weights from the oracle (with drops)."""
    I = gen.make_inputs("tiny", T=T, H=64, F=32, E=E, k=4, dtype="bf16", seed=92, drop=0.1)
    r = oracle.route(I.f64(I.x), I.f64(I.Wr), None, I.k, I.drop)
    dref = oracle.dispatch(r.ids, r.keep, I.E)
    x = gen.storage_to_torch(I.x, "bf16").to(dev)
    ids = torch.from_numpy(r.ids.astype(np.int32)).to(dev)
    w = torch.from_numpy(r.w.astype(np.float32)).to(dev)
    x_perm, off, row_token, inv = moe.moe_permute(x, ids, w, I.E)
    torch.cuda.synchronize()
    g = dict(ids=ids, w=w, off=off, row_token=row_token, inv=inv, x_perm=x_perm)
    check_routing(g, r, dref, I.x)


@pytest.mark.parametrize("T,H,E,k,drop,zipf", [
    (32, 2048, 128, 8, 0.0, 0.0),     # decode shape: maps built by the router's reduction launch (32 splits)
    (128, 1024, 256, 8, 0.0, 0.0),    # 1024 assignments, the fused limit; 16 splits, 256 padded experts
    (1, 4096, 32, 4, 0.0, 0.0),       # one token, 64 splits, 32 padded experts
    (20, 2048, 64, 6, 0.1, 1.2),      # drops and a skewed bias
    (200, 1024, 64, 4, 0.0, 0.0),     # 7 token blocks x 16 splits
    (100, 256, 64, 4, 0.0, 0.0),      # 4 splits: router, then the one-workgroup dispatch
    (3000, 128, 256, 8, 0.05, 0.0),   # 24,000 assignments: two-pass dispatch
    (9000, 64, 1000, 4, 0.0, 1.2),    # 36 chunks x 1000 experts: count / scan / index
])
def test_forward_routing_maps(dev, T, H, E, k, drop, zipf):
    """moe_forward's own routing outputs (ids, weights, offsets, inverse map) bit-exact against the oracle on
    every dispatch path, and y within the layer bound."""
    I = gen.make_inputs("tiny", T=T, H=H, F=64, E=E, k=k, dtype="bf16", seed=4000 + T, drop=drop, zipf=zipf)
    _say(f"case T={T} H={H} E={E} k={k} drop={drop} zipf={zipf}")
    d = gen.to_device(I, dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    inv = torch.empty((T, k), dtype=torch.int32, device=dev)
    y = None
    for _ in range(2):  # a second call on the same buffers: the hand-off state carries nothing over
        y = moe.moe_forward(d["x"], d["Wr"], d["bias"], d["W1"], d["W2"], k, I.drop, topk_ids=ids, topk_w=w,
                            expert_offsets=off, inv=inv)
    torch.cuda.synchronize()
    ref = oracle.forward(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), I.f64(I.W1()), I.f64(I.W2()), k, I.drop)
    assert np.array_equal(ids.cpu().numpy(), ref.route.ids), "expert ids differ"
    assert np.abs(w.cpu().numpy().astype(np.float64) - ref.route.w).max() <= W_TOL
    assert np.array_equal(off.cpu().numpy(), ref.dispatch.offsets), "expert offsets differ"
    assert np.array_equal(inv.cpu().numpy(), ref.dispatch.inv), "inverse map differs"
    check_y(y.double().cpu().numpy(), ref.y)


@pytest.mark.parametrize("T,H,F,E,k,zipf", [
    (300, 256, 256, 5, 2, 0.0),      # ragged 64-row tiles, one 256-column chunk per phase
    (700, 512, 512, 8, 2, 1.2),      # skewed groups (some experts empty), two chunks of F
    (1024, 256, 768, 4, 3, 0.0),     # F = 768: the largest h (64 x 768 bf16 = 96 KB of LDS)
    (37, 256, 256, 16, 4, 0.0),      # few rows: most groups below one tile, some empty
])
def test_grouped_ffn_fused(dev, T, H, F, E, k, zipf):
    """The one-launch grouped FFN with h kept in LDS: y_perm against the oracle (layer bound) and against the
    two-launch moe_grouped_ffn, which rounds h to bf16 the same way and accumulates every output over k in the
    same order (printed: the largest difference)."""
    I = gen.make_inputs("tiny", T=T, H=H, F=F, E=E, k=k, dtype="bf16", seed=5000 + T, zipf=zipf)
    _say(f"case T={T} H={H} F={F} E={E} k={k} zipf={zipf}")
    d = gen.to_device(I, dev)
    ids, w = moe.moe_route(d["x"], d["Wr"], d["bias"], k, I.drop)
    x_perm, off, row_token, inv = moe.moe_permute(d["x"], ids, w, E)
    y_two, _ = moe.moe_grouped_ffn(x_perm, off, d["W1"], d["W2"], T, k)
    y_one = moe.moe_grouped_ffn_fused(x_perm, off, d["W1"], d["W2"], T, k)
    torch.cuda.synchronize()
    A = int(off[-1].item())
    ref = oracle.forward(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), I.f64(I.W1()), I.f64(I.W2()), k, I.drop)
    check_y(y_one[:A].double().cpu().numpy(), ref.y_perm[:A])
    diff = float((y_one[:A] - y_two[:A]).abs().max()) if A else 0.0
    scale = float(y_two[:A].abs().max()) if A else 1.0
    _say(f"fused vs two-launch: max |diff| {diff:.3e} (max |y_perm| {scale:.3e})")
    assert diff <= 1e-5 * scale


# ------------------------------------------- block-scaled fp16 extremes --
def test_scaled16_dynamic_range(dev):
    """The one-call layer's block-scaled fp16 y_perm at the ends of its range. W2 columns are scaled so that
    y_perm has, per 32-column block: one column 1e-12 below the rest (it falls under fp16's normal range after
    scaling), a block near 1e-36 (its exponent clamps at -127), a block near 1e20, an all-zero block (s = 0),
    and ordinary blocks. The one-call result must stay within the element-wise rounding bound of the step-wise
    (fp32 y_perm) result. The step-wise result meets the usual bar of the oracle on each block at its own scale
    (the ordinary columns, and the 1e20 block alone); the 1e-36 block is left out of that comparison, since most
    of its bf16 weights are subnormal, which the matrix cores may flush to zero."""
    I = gen.make_inputs("tiny", T=600, H=256, F=256, E=4, k=2, dtype="bf16", seed=151)  # 256-row tiles, packed W2
    d = gen.to_device(I, dev)
    colscale = torch.ones(I.H, dtype=torch.float32)
    colscale[5] = 1e-12
    colscale[32:64] = 1e-36
    colscale[64:96] = 1e20
    colscale[96:128] = 0.0
    d["W2"] = (d["W2"].float() * colscale.to(dev)).to(torch.bfloat16)
    g = run_steps(d, I, dev)
    A = int(g["off"][-1].item())
    y1 = moe.moe_forward(d["x"], d["Wr"], d["bias"], d["W1"], d["W2"], I.k, I.drop)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y1).all())
    assert bool((y1[:, 96:128] == 0).all())
    bound = scaled16_bound(g["y_perm"], A, g["inv"], g["w"], g["y"])
    assert bool(((y1 - g["y"]).abs().double() <= bound).all()), "one-call y outside the fp16 rounding bound"
    W2 = d["W2"].float().double().cpu().numpy()
    ref = oracle.forward(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), I.f64(I.W1()), W2, I.k, I.drop)
    check_routing(g, ref.route, ref.dispatch)
    y = g["y"].double().cpu().numpy()
    for cols in (np.r_[0:32, 128:256], np.r_[64:96]):
        check_y(y[:, cols], ref.y[:, cols])


# ---------------------------------------------------------- exact ties --
@pytest.mark.parametrize("T,E,k", [
    (512, 16, 4),      # H loop split across workgroups, top-k in the reduction kernel
    (16384, 16, 4),    # enough token blocks: no split, top-k fused into the router kernel
    (512, 256, 8),     # four logits per lane
    (8192, 128, 8),    # 64 tokens per workgroup sharing each Wr stage, split H loop
    (16384, 64, 4),    # 64 tokens per workgroup, top-k fused into the router kernel
])
def test_router_exact_ties(dev, T, E, k):
    """Experts with identical router columns get bit-identical logits on both sides (each logit is the same
    ordered sum of the same products); where such a tie straddles the k-th place, the lower expert id must be
    selected. Tokens whose k-th/(k+1)-th gap is neither exactly 0 (a planted tie) nor clear of fp32 rounding
    (>= 1e-4) are left out; the test requires some tokens with a tie at the boundary."""
    H = 256
    I = gen.make_inputs("tiny", T=T, H=H, F=64, E=E, k=k, dtype="bf16", seed=141 + E)
    _say(f"case ties T={T} E={E} k={k}")
    pairs = [(5, 3), (9, 3), (12, 0), (13, 7)] + ([(2 * i + 1, 2 * i) for i in range(8, 64)] if E >= 128 else [])
    Wr = I.Wr.copy()
    for dst, src in pairs:
        Wr[:, dst] = Wr[:, src]
    ids, w = moe.moe_route(gen.storage_to_torch(I.x, I.dtype).to(dev), gen.storage_to_torch(Wr, I.dtype).to(dev),
                           None, k)
    torch.cuda.synchronize()
    lg = oracle.router_logits(I.f64(I.x), I.f64(Wr))
    for dst, src in pairs:
        lg[:, dst] = lg[:, src]  # exact ties in fp64 too, whatever the matrix product's summation order
    ids_ref, gap = oracle.select_topk(lg, k)
    w_ref, _ = oracle.selection_weights(lg, ids_ref)
    tied = gap == 0.0
    use = tied | (gap >= 1e-4)
    assert int(tied.sum()) >= 5, "no tie at the k-th place: the case does not test the rule"
    assert np.array_equal(ids.cpu().numpy()[use], ids_ref[use])
    assert np.abs(w.cpu().numpy().astype(np.float64)[use] - w_ref[use]).max() <= W_TOL
    _say(f"ties at the k-th place: {int(tied.sum())} of {T} tokens; compared {int(use.sum())}")


@pytest.mark.parametrize("T,H,F,E,k", [
    (256, 128, 64, 16, 4),    # register-staged grouped FFN, fp32 y_perm
    (600, 256, 256, 4, 2),    # direct-to-LDS large tiles, k-blocked h, block-scaled fp16 y_perm
    (40, 256, 256, 16, 4),    # weight-streaming tiles, block-scaled fp16 y_perm
])
def test_bf16_output_and_determinism(dev, T, H, F, E, k):
    I = gen.make_inputs("tiny", T=T, H=H, F=F, E=E, k=k, dtype="bf16", seed=93)
    d = gen.to_device(I, dev)
    a = moe.moe_forward(d["x"], d["Wr"], None, d["W1"], d["W2"], I.k)
    b = moe.moe_forward(d["x"], d["Wr"], None, d["W1"], d["W2"], I.k)
    c = moe.moe_forward(d["x"], d["Wr"], None, d["W1"], d["W2"], I.k, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a, b)  # bit-identical reruns
    assert torch.equal(c, a.to(torch.bfloat16))  # bf16 output = RNE of the fp32 accumulator


# ------------------------------------------------------ full workloads --
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "mixtral_shared", "skew"])
def test_full_workload(dev, name):
    """Every workload at its full size, every token: the fp64 oracle runs the whole layer (expert weights fetched
    one expert at a time, so host memory stays bounded) and both the one-call and the step-wise GPU results are
    compared with it element by element: routing arrays bit-exact, y_perm and y within 2e-2 * rms (layer
    definition: page 3, section "MoE层的结构与token路由")."""
    I = gen.make_inputs(name)
    _say(f"case {name}: T={I.T} H={I.H} F={I.F} E={I.E} k={I.k} Fs={I.Fs} drop={I.drop}")
    d = gen.to_device(I, dev, keep_host=True)
    W1h, W2h = d.pop("W1_host"), d.pop("W2_host")
    ids = torch.empty((I.T, I.k), dtype=torch.int32, device=dev)
    w = torch.empty((I.T, I.k), dtype=torch.float32, device=dev)
    off1 = torch.empty(I.E + 1, dtype=torch.int32, device=dev)
    inv1 = torch.empty((I.T, I.k), dtype=torch.int32, device=dev)
    y = moe.moe_forward(d["x"], d["Wr"], d["bias"], d["W1"], d["W2"], I.k, I.drop, W1s=d["W1s"], W2s=d["W2s"],
                        topk_ids=ids, topk_w=w, expert_offsets=off1, inv=inv1)
    g = run_steps(d, I, dev)
    # the one-call dispatch maps (built inside the router launch at decode) equal the step-wise ones
    assert torch.equal(g["ids"], ids) and torch.equal(g["off"], off1) and torch.equal(g["inv"], inv1)
    A = int(g["off"][-1].item())
    # moe_forward keeps y_perm as block-scaled fp16: within 2^-10 * max|y_perm| of the step-wise (fp32 y_perm) result
    assert float((g["y"] - y).abs().max()) <= 2.0 ** -10 * float(g["y_perm"][:A].abs().max())
    y_one = y.double().cpu().numpy()
    y_steps = g["y"].double().cpu().numpy()
    y_perm = g["y_perm"][:A].double().cpu().numpy()
    del d, y, ids, w
    g = {k_: v for k_, v in g.items() if k_ not in ("y", "y_perm")}
    torch.cuda.empty_cache()

    def W1(e):
        return I.f64(W1h[e])

    def W2(e):
        return I.f64(W2h[e])

    ref = oracle.forward(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), W1, W2, I.k, I.drop, I.f64(I.W1s()), I.f64(I.W2s()))
    check_routing(g, ref.route, ref.dispatch, I.x)
    rel_perm = check_y(y_perm, ref.y_perm[:A])
    rel_one = check_y(y_one, ref.y)
    rel_steps = check_y(y_steps, ref.y)
    _say(f"{name}: routing bit-exact over {I.T} tokens; all {I.T} tokens of y compared: max-abs/rms one-call "
         f"{rel_one:.3e}, step-wise {rel_steps:.3e}; y_perm ({A} rows) {rel_perm:.3e}")


# ---------------------------------------------- one very large expert --
def test_group_beyond_32bit_bytes(dev):
    """One expert holding 131,072 rows of H = 8192: its fp32 y_perm spans 4 GiB, more than a 32-bit byte count
    measured from the group's first row. Every GEMM epilogue must bound its stores by its own tile's rows; the
    first tiles of the group (tokens 0..255 among the samples) would otherwise lose or misplace their stores.
    Step-wise and one-call y are checked against the oracle on sampled tokens (E = 1, k = 1: weight 1). The
    inputs are seeded torch normals drawn on the device (the shared generator would take a minute here)."""
    import types
    T, H, F = 131072, 8192, 64
    _say(f"case one-group T={T} H={H} F={F}")
    gdev = torch.Generator(device=dev).manual_seed(131)
    gcpu = torch.Generator().manual_seed(132)
    d = {"x": torch.randn((T, H), generator=gdev, device=dev).to(torch.bfloat16),
         "Wr": (torch.randn((H, 1), generator=gcpu) / H ** 0.5).to(torch.bfloat16).to(dev),
         "W1": (torch.randn((1, H, F), generator=gcpu) / H ** 0.5).to(torch.bfloat16).to(dev),
         "W2": (torch.randn((1, F, H), generator=gcpu) / F ** 0.5).to(torch.bfloat16).to(dev),
         "bias": None, "W1s": None, "W2s": None}
    I = types.SimpleNamespace(T=T, k=1, E=1, Fs=0, drop=0.0)
    g = run_steps(d, I, dev)
    assert bool((g["ids"] == 0).all()) and int(g["off"][-1].item()) == T
    y1 = moe.moe_forward(d["x"], d["Wr"], None, d["W1"], d["W2"], 1)
    torch.cuda.synchronize()
    toks = np.array(sorted({0, 1, 100, 255, 256, 511, 4096, 65535, 65536, 100000, T - 257, T - 1}))
    sel = torch.from_numpy(toks).to(dev)

    def f64(t):
        return t.float().double().cpu().numpy()

    W1, W2 = f64(d["W1"][0]), f64(d["W2"][0])
    _, _, _, yref = oracle.forward_tokens(np.arange(len(toks)), f64(d["x"][sel]), f64(d["Wr"]), np.zeros(1),
                                          lambda e: W1, lambda e: W2, 1)
    check_y(g["y"][sel].double().cpu().numpy(), yref)
    check_y(y1[sel].double().cpu().numpy(), yref)


# ------------------------------------------------ no kept assignments --
def test_nothing_kept(dev):
    """A batch whose every slot is dropped (weight 0) or names no expert: permute keeps no row (all offsets 0,
    inv all -1, row_token and x_perm untouched), the grouped FFN over zero rows writes nothing, and the combine
    gives 0 (or exactly the shared expert's row)."""
    T, H, F, E, k = 12, 64, 64, 4, 3
    x = torch.randn((T, H), device=dev).to(torch.bfloat16)
    ids = torch.tensor([[0, 1, 2], [5, -1, 4]] * (T // 2), dtype=torch.int32, device=dev)  # even: dropped; odd: no such expert
    w = torch.zeros((T, k), dtype=torch.float32, device=dev)
    w[1::2] = 0.5                                   # odd tokens: nonzero weights, but every id is out of range
    sentinel = torch.full((T * k, H), 7.0, device=dev).to(torch.bfloat16)
    x_perm = sentinel.clone()
    off = torch.full((E + 1,), 99, dtype=torch.int32, device=dev)
    row_token = torch.full((T * k,), -5, dtype=torch.int32, device=dev)
    inv = torch.full((T, k), 99, dtype=torch.int32, device=dev)
    moe.moe_permute(x, ids, w, E, x_perm=x_perm, expert_offsets=off, row_token=row_token, inv=inv)
    torch.cuda.synchronize()
    assert torch.equal(off, torch.zeros_like(off))
    assert torch.equal(inv, torch.full_like(inv, -1))
    assert torch.equal(row_token, torch.full_like(row_token, -5)) and torch.equal(x_perm, sentinel)

    W1 = (torch.randn((E, H, F), device=dev) / 8).to(torch.bfloat16)
    W2 = (torch.randn((E, F, H), device=dev) / 8).to(torch.bfloat16)
    y_perm = torch.full((T * k, H), 3.0, device=dev)
    moe.moe_grouped_ffn(x_perm, off, W1, W2, T, k, y_perm=y_perm)
    torch.cuda.synchronize()
    assert torch.equal(y_perm, torch.full_like(y_perm, 3.0))

    y = moe.moe_combine(y_perm, inv, w)
    y_sh = torch.randn((T, H), device=dev)
    y2 = moe.moe_combine(y_perm, inv, w, y_shared=y_sh)
    torch.cuda.synchronize()
    assert torch.equal(y, torch.zeros_like(y))
    assert torch.equal(y2, y_sh)
