"""HIP graph capture of the one-call layers.

The library enqueues kernels only (no allocation, memset or synchronisation),
so a whole layer can be captured once and replayed. Each case captures the
layer with its workspace and outputs allocated beforehand, replays it three
times with unrelated eager calls of the library and synchronisations in
between, and requires every replay to equal the eager result bit for bit; a
fourth replay after new data is copied into the captured input must equal an
eager call on that data (the graph reads its inputs at replay time).
"""
import pytest

import gen

torch = pytest.importorskip("torch")
moe = pytest.importorskip("top_routing_grouped_gemm_amd")

pytestmark = pytest.mark.gpu

CASES = [
    # name, sizes, path
    ("decode-bf16", dict(T=32, H=256, F=256, E=16, k=4, seed=701), "bf16"),   # weight-streaming tiles
    ("prefill-bf16", dict(T=600, H=256, F=256, E=4, k=2, seed=702), "bf16"),  # 256x256 tiles, k-blocked h
    ("drop-shared", dict(T=64, H=128, F=128, E=8, k=2, seed=703, drop=0.2, Fs=64), "bf16"),
    ("shared-in-routed-launches", dict(T=600, H=256, F=256, E=4, k=2, seed=707, Fs=256), "bf16"),  # Fs == F
    ("decode-fp8", dict(T=32, H=256, F=256, E=16, k=4, seed=704), "fp8"),
    ("prefill-mx", dict(T=600, H=256, F=256, E=4, k=2, seed=705), "mx"),
    ("large-batch", dict(T=4096, H=256, F=256, E=64, k=4, seed=706), "bf16"),  # 64-token router workgroups,
                                                                              # several dispatch chunks
]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    return torch.device("cuda:0")


def _layer(path, d, I, dev):
    """A closure running the one-call layer of `path` on tensors held in d (x is read at call time)."""
    k, drop = I.k, I.drop
    T, H = I.T, I.H
    if path == "bf16":
        ws = torch.empty(max(moe.moe_workspace_bytes(T, H, I.F, I.E, k, I.Fs, d["x"].dtype), 1), dtype=torch.uint8,
                         device=dev)
        y = torch.empty((T, H), dtype=torch.float32, device=dev)

        def run(x):
            return moe.moe_forward(x, d["Wr"], d["bias"], d["W1"], d["W2"], k, drop, W1s=d["W1s"], W2s=d["W2s"],
                                   y=y, ws=ws)
        return run
    if path == "fp8":
        W1q, s1 = moe.moe_quantize_fp8(d["W1"])
        W2q, s2 = moe.moe_quantize_fp8(d["W2"])
        lib = moe.load_library()
        ws = torch.empty(lib.moe_workspace_bytes(T, H, I.F, I.E, k, 0, moe.MOE_BF16), dtype=torch.uint8, device=dev)
        y = torch.empty((T, H), dtype=torch.float32, device=dev)

        def run(x):
            return moe.moe_forward_fp8(x, d["Wr"], d["bias"], W1q, s1, W2q, s2, k, drop, y=y, ws=ws)
        return run
    W1q, W1s_ = moe.moe_quantize_mxfp8(d["W1"])
    W2q, W2s_ = moe.moe_quantize_mxfp8(d["W2"])
    lib = moe.load_library()
    ws = torch.empty(lib.moe_mxfp8_workspace_bytes(T, H, I.F, I.E, k), dtype=torch.uint8, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)

    def run(x):
        return moe.moe_forward_mxfp8(x, d["Wr"], d["bias"], W1q, W1s_, W2q, W2s_, I.F, k, drop, y=y, ws=ws)
    return run


@pytest.mark.parametrize("name,sizes,path", CASES, ids=[c[0] for c in CASES])
def test_graph_replay(dev, name, sizes, path):
    print(f"case {name} {sizes} {path}", flush=True)
    I = gen.make_inputs("tiny", dtype="bf16", **sizes)
    d = gen.to_device(I, dev)
    I2 = gen.make_inputs("tiny", dtype="bf16", **dict(sizes, seed=sizes["seed"] + 50))
    x2 = gen.to_device(I2, dev)["x"]

    run = _layer(path, d, I, dev)            # captured: its own workspace and output
    other = _layer(path, d, I, dev)          # eager calls in between: another workspace and output
    x_static = d["x"].clone()
    eager = run(x_static).clone()
    eager2 = other(x2).clone()
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):            # warm-up on the capture stream's side
        run(x_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_graph = run(x_static)
    torch.cuda.synchronize()

    for rep in range(3):
        y_graph.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph, eager), f"replay {rep} differs from the eager call"
        other(x2)                            # unrelated library work between replays
        torch.cuda.synchronize()
    x_static.copy_(x2)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y_graph, eager2), "replay on new input data differs from the eager call on it"
