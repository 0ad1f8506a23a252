"""The no-allocation forward (moe_forward_noalloc) against moe_forward, through the C ABI.

Both run the same kernels, the first in the library's static per-GPU scratch array, the second in a caller
workspace, so y and every debug output must be bit-identical. Two calls in a row, the second smaller than the
first (the array keeps the first call's contents), then one that mixes tile regimes with a shared expert and a
drop threshold; a batch whose buffers do not fit the array is refused before anything is launched.
"""
import numpy as np
import pytest

import gen
import oracle

torch = pytest.importorskip("torch")
moe = pytest.importorskip("top_routing_grouped_gemm_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    return torch.device("cuda:0")


def _both(d, I, dev):
    T, k, E = I.T, I.k, I.E
    outs = []
    for fn in (moe.moe_forward, moe.moe_forward_noalloc):
        ids = torch.full((T, k), -7, dtype=torch.int32, device=dev)
        w = torch.full((T, k), -7.0, dtype=torch.float32, device=dev)
        off = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
        inv = torch.full((T, k), -7, dtype=torch.int32, device=dev)
        y = fn(d["x"], d["Wr"], d["bias"], d["W1"], d["W2"], k, I.drop, W1s=d["W1s"], W2s=d["W2s"], topk_ids=ids,
               topk_w=w, expert_offsets=off, inv=inv)
        outs.append((y, ids, w, off, inv))
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("name,over", [
    ("decode", {}),                                                   # the full decode layer: weight-streaming tiles
    ("decode", {"T": 5, "H": 256, "F": 128, "E": 16, "k": 4}),        # smaller, right after
    ("tiny", {"T": 300, "H": 256, "F": 256, "E": 12, "k": 3, "dtype": "bf16", "Fs": 128, "drop": 0.2,
              "zipf": 1.2}),                                          # mixed regimes, shared expert, drop
    ("tiny", {"T": 600, "H": 256, "F": 256, "E": 4, "k": 2, "dtype": "bf16", "Fs": 256}),  # shared expert in the
                                                                                            # routed launches
])
def test_noalloc_matches_forward(dev, name, over):
    I = gen.make_inputs(name, **over)
    print(f"case noalloc {name} {over}", flush=True)
    d = gen.to_device(I, dev)
    (y0, ids0, w0, off0, inv0), (y1, ids1, w1, off1, inv1) = _both(d, I, dev)
    for a, b, what in ((ids0, ids1, "ids"), (w0, w1, "weights"), (off0, off1, "offsets"), (inv0, inv1, "inv"),
                       (y0, y1, "y")):
        assert torch.equal(a, b), f"{what} differ from moe_forward"
    # and the routing is the oracle's (the scratch path is a full layer, not a copy of a stale result)
    r = oracle.route(I.f64(I.x), I.f64(I.Wr), I.bias_f64(), I.k, I.drop)
    assert np.array_equal(ids1.cpu().numpy(), r.ids)


def test_noalloc_refuses_oversized(dev):
    I = gen.make_inputs("tiny", T=8192, H=2048, F=768, E=16, k=8, dtype="bf16")
    x = torch.zeros((I.T, I.H), dtype=torch.bfloat16, device=dev)
    Wr = torch.zeros((I.H, I.E), dtype=torch.bfloat16, device=dev)
    W1 = torch.zeros((I.E, I.H, I.F), dtype=torch.bfloat16, device=dev)
    W2 = torch.zeros((I.E, I.F, I.H), dtype=torch.bfloat16, device=dev)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_noalloc(x, Wr, None, W1, W2, I.k)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
