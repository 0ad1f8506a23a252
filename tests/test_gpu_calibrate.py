"""The measurement aids run and write their sinks (no results to check beyond finiteness: they time the chip)."""
import pytest
import torch

import top_routing_grouped_gemm_amd as moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()
    return torch.device("cuda:0")


def test_calibration_kernels_run(dev):
    src = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    sink = torch.full((16 * 512,), float("nan"), dtype=torch.float32, device=dev)
    for mode in (0, 1, 2):
        moe.moe_calibrate_gemm_kstep(mode, 16, 8, src=src if mode else None, sink=sink)
        torch.cuda.synchronize()
        if mode >= 1:  # zero operands: every accumulator (mode 1) or the LDS byte (mode 2) reads back 0
            assert bool((sink == 0).all()), f"mode {mode}"
    sink2 = torch.empty(4 * 4 * 64, dtype=torch.float32, device=dev)
    assert moe.moe_calibrate_mfma_bf16(4, 4, 16, sink2) == 4 * 4 * 16 * 8 * 32768
    torch.cuda.synchronize()
    assert bool(torch.isfinite(sink2).all())
    assert moe.moe_calibrate_mfma_bf16(4, 4, 16, sink2, random_operands=True) == 4 * 4 * 16 * 8 * 32768
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    assert moe.moe_calibrate_stream_read(buf, 8) == 1 << 20
    torch.cuda.synchronize()
    assert bool(torch.isfinite(sink2).all())
